"""The five seeded workloads and a generic recipe for smaller test shapes.

Draw order inside one workload (a numpy PCG64 stream per seed; the two pool
fills come from their own keyed streams, see _pool_bits):
context lengths -> physical block permutation -> q -> pool K -> pool V ->
new k, v.  Nothing here knows how a token is laid out inside a cache block:
the pools are returned as flat arrays of independent N(0,1) values, one per
element, so any layout reads the same distribution.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BLOCK_SIZE = 16
# Block-table entries past a sequence's used blocks hold this value: an index no
# pool ever has, so a kernel that read one would fault or fail a check.
TABLE_SENTINEL = np.int32(0x7FFFFFFF)

CONFIG_NAMES = {
    1: "tiny-fp32-mha",
    2: "7b-shape-b64-bf16",
    3: "gqa-b256-bf16",
    4: "long-context-split-bf16",
    5: "shared-prefix-50-step-bf16",
}


def bits_dtype(dtype: str):
    """numpy container type for one element's bit pattern."""
    if dtype == "bf16":
        return np.uint16
    if dtype == "f32":
        return np.uint32
    if dtype in ("fp8", "int8"):
        return np.uint8
    raise ValueError(f"unsupported dtype {dtype!r}")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return bits.

    Inputs here are finite N(0,1) draws, so no NaN/Inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)            # the bit that breaks ties towards even
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _normal_bits(rng: np.random.Generator, n: int, dtype: str,
                 chunk: int = 1 << 24) -> np.ndarray:
    """n independent N(0,1) values as bit patterns, drawn from `rng` in order."""
    out = np.empty(n, dtype=bits_dtype(dtype))
    buf = np.empty(min(chunk, max(n, 1)), dtype=np.float32)
    pos = 0
    while pos < n:
        m = min(chunk, n - pos)
        rng.standard_normal(out=buf[:m], dtype=np.float32)
        out[pos:pos + m] = f32_to_bf16_bits(buf[:m]) if dtype == "bf16" else buf[:m].view(np.uint32)
        pos += m
    return out


POOL_CHUNK = 1 << 22  # elements per independently keyed stream of a pool fill


FP8_MAG_CODES = 0x40  # fp8 pool bytes: magnitude codes 0x00..0x3F
INT8_CODE_SD = 40.0   # int8 pool codes: rint(40 N(0,1)) clipped to +-127
INT8_SCALE_RANGE = (0.02, 0.03)  # int8 pool row scales: uniform on this range


def _pool_bits(seed: int, tag: int, n: int, dtype: str, threads: int = 0) -> np.ndarray:
    """A pool's n values, drawn in fixed chunks of POOL_CHUNK elements.

    bf16 / f32: N(0,1) values.  fp8: bytes with a random sign bit and a
    magnitude code drawn uniformly from 0x00..0x3F (in the E4M3 format those
    are the values 0 to 1.875, spaced logarithmically; no NaN code is drawn).
    int8: codes rint(40 N(0,1)) clipped to +-127 (the row scales come from
    kv_pool, which appends them).
    Chunk i comes from its own PCG64 stream keyed by SeedSequence([seed, tag, i]),
    so the values do not depend on how many threads fill them.
    """
    out = np.empty(n, dtype=bits_dtype(dtype))
    nchunks = -(-n // POOL_CHUNK)

    def fill(i: int) -> None:
        lo = i * POOL_CHUNK
        m = min(POOL_CHUNK, n - lo)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, i])))
        if dtype == "int8":
            g = rng.standard_normal(m, dtype=np.float32) * np.float32(INT8_CODE_SD)
            out[lo:lo + m] = np.clip(np.rint(g), -127, 127).astype(np.int8).view(np.uint8)
            return
        if dtype == "fp8":
            r = rng.integers(0, 2 * FP8_MAG_CODES, size=m, dtype=np.uint8)
            out[lo:lo + m] = (r & np.uint8(FP8_MAG_CODES - 1)) | ((r & np.uint8(FP8_MAG_CODES)) << np.uint8(1))
            return
        buf = rng.standard_normal(m, dtype=np.float32)
        out[lo:lo + m] = f32_to_bf16_bits(buf) if dtype == "bf16" else buf.view(np.uint32)

    threads = threads or min(16, os.cpu_count() or 1)
    if nchunks <= 1 or threads <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def kv_pool(seed: int, tag: int, num_blocks: int, H_kv: int, d: int, dtype: str) -> np.ndarray:
    """One cache buffer of a pool: num_blocks*H_kv*16*d elements; an int8 cache
    also holds one float32 scale per (block, head, slot) row after its codes,
    drawn uniformly from INT8_SCALE_RANGE (so values code * scale are near
    N(0,1))."""
    n = num_blocks * H_kv * BLOCK_SIZE * d
    codes = _pool_bits(seed, tag, n, dtype)
    if dtype != "int8":
        return codes
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, 1 << 30])))
    scales = rng.uniform(*INT8_SCALE_RANGE, size=num_blocks * H_kv * BLOCK_SIZE).astype(np.float32)
    return np.concatenate([codes, scales.view(np.uint8)])


@dataclass
class DecodeStep:
    """Inputs of one decode step: one new token per sequence.

    context_lens[b] counts every cached token of sequence b *including* the one
    this step writes, so the new token sits at position context_lens[b] - 1.
    """
    context_lens: np.ndarray      # int32 [B]
    q: np.ndarray                 # bits [B, H, d]
    new_k: np.ndarray             # bits [B, H_kv, d]
    new_v: np.ndarray             # bits [B, H_kv, d]


@dataclass
class MultiStep:
    """Inputs of one step with several new tokens per sequence (a prefill chunk
    or a block of draft tokens to verify): sequence b's rows are
    query_start[b] .. query_start[b+1]-1, the tokens at positions
    context_lens[b] - n_b .. context_lens[b] - 1 (context_lens count them)."""
    context_lens: np.ndarray      # int32 [B]
    query_start: np.ndarray       # int32 [B + 1]
    q: np.ndarray                 # bits [T, H, d]
    new_k: np.ndarray             # bits [T, H_kv, d]
    new_v: np.ndarray             # bits [T, H_kv, d]


@dataclass
class Workload:
    name: str
    dtype: str                    # activations (q, out, new rows): "f32" | "bf16"
    B: int
    H: int
    H_kv: int
    d: int
    num_blocks: int
    max_nb: int                   # columns of the block table
    scale: float
    partition_size: int           # 0 = single pass, else tokens per split
    block_tables: np.ndarray      # int32 [B, max_nb]; unused entries = TABLE_SENTINEL
    k_pool: np.ndarray            # bits, flat, num_blocks*H_kv*16*d elements
    v_pool: np.ndarray
    steps: List[DecodeStep] = field(default_factory=list)
    block_size: int = BLOCK_SIZE
    seed: int = 0
    multi: Optional[MultiStep] = None  # a several-token step, if the workload has one
    kv_dtype: Optional[str] = None  # cache elements: as dtype, or "fp8" (E4M3 codes)
    k_scale: float = 1.0            # per-tensor scales of an fp8 cache
    v_scale: float = 1.0

    def __post_init__(self):
        if self.kv_dtype is None:
            self.kv_dtype = self.dtype

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_dtype in ("fp8", "int8") else self.elem_bytes

    @property
    def kv_row_extra_bytes(self) -> int:
        """Bytes stored per cached (token, KV head) row besides its elements:
        an int8 cache's float32 row scale."""
        return 4 if self.kv_dtype == "int8" else 0

    @property
    def group(self) -> int:
        return self.H // self.H_kv

    @property
    def pool_elems(self) -> int:
        return self.num_blocks * self.H_kv * self.block_size * self.d

    @property
    def max_context_len(self) -> int:
        return int(max(int(s.context_lens.max()) for s in self.steps))


def _blocks_for(n_tokens: int) -> int:
    return -(-int(n_tokens) // BLOCK_SIZE)


def scattered_workload(name: str, dtype: str, B: int, H: int, H_kv: int, d: int,
                       context_lens: Sequence[int], seed: int, rng=None,
                       pool_factor: float = 1.25, max_nb: Optional[int] = None,
                       partition_size: int = 0, num_blocks: Optional[int] = None,
                       kv_dtype: Optional[str] = None, k_scale: float = 1.0,
                       v_scale: float = 1.0) -> Workload:
    """One decode step over sequences whose blocks are scattered at random.

    The pool holds ceil(pool_factor * total blocks) blocks (or num_blocks); the
    physical blocks are the first sum(nb) entries of a seeded permutation of the
    pool, dealt to the sequences in order.
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(context_lens, dtype=np.int64)
    if ctx.shape != (B,):
        raise ValueError("need one context length per sequence")
    nb = [_blocks_for(c) for c in ctx]
    total = int(sum(nb))
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * total)), 1)
    if num_blocks < total:
        raise ValueError("pool smaller than the blocks the sequences need")
    if max_nb is None:
        max_nb = max(max(nb), 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((B, max_nb), TABLE_SENTINEL, dtype=np.int32)
    pos = 0
    for b in range(B):
        tables[b, :nb[b]] = perm[pos:pos + nb[b]]
        pos += nb[b]
    q = _normal_bits(rng, B * H * d, dtype).reshape(B, H, d)
    kv_dtype = kv_dtype or dtype
    k_pool = kv_pool(seed, 1, num_blocks, H_kv, d, kv_dtype)
    v_pool = kv_pool(seed, 2, num_blocks, H_kv, d, kv_dtype)
    new_k = _normal_bits(rng, B * H_kv * d, dtype).reshape(B, H_kv, d)
    new_v = _normal_bits(rng, B * H_kv * d, dtype).reshape(B, H_kv, d)
    step = DecodeStep(context_lens=ctx.astype(np.int32), q=q, new_k=new_k, new_v=new_v)
    return Workload(name=name, dtype=dtype, B=B, H=H, H_kv=H_kv, d=d,
                    num_blocks=num_blocks, max_nb=max_nb, scale=1.0 / math.sqrt(d),
                    partition_size=partition_size, block_tables=tables,
                    k_pool=k_pool, v_pool=v_pool, steps=[step], seed=seed,
                    kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale)


def add_multi_step(w: Workload, query_lens: Sequence[int], rng=None, seed: int = 0) -> Workload:
    """Give w a step of query_lens[b] new tokens per sequence: the last
    query_lens[b] of its first step's context (q [T, H, d], new K/V rows
    [T, H_kv, d] drawn in that order from rng, or from a PCG64 stream of seed)."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(w.steps[0].context_lens, dtype=np.int32)
    qlen = np.asarray(query_lens, dtype=np.int64)
    if qlen.shape != (w.B,):
        raise ValueError("need one query length per sequence")
    qs = np.zeros(w.B + 1, dtype=np.int32)
    qs[1:] = np.cumsum(qlen)
    T = int(qs[-1])
    w.multi = MultiStep(context_lens=ctx, query_start=qs,
                        q=_normal_bits(rng, T * w.H * w.d, w.dtype).reshape(T, w.H, w.d),
                        new_k=_normal_bits(rng, T * w.H_kv * w.d, w.dtype).reshape(T, w.H_kv, w.d),
                        new_v=_normal_bits(rng, T * w.H_kv * w.d, w.dtype).reshape(T, w.H_kv, w.d))
    return w


def multi_token_workload(name: str, dtype: str, B: int, H: int, H_kv: int, d: int,
                         context_lens: Sequence[int], query_lens: Sequence[int], seed: int,
                         kv_dtype: Optional[str] = None, k_scale: float = 1.0,
                         v_scale: float = 1.0, max_nb: Optional[int] = None) -> Workload:
    """A scattered pool as scattered_workload, plus a step of query_lens[b] new
    tokens per sequence (the last query_lens[b] of its context_lens[b])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = scattered_workload(name, dtype, B, H, H_kv, d, context_lens, seed, rng=rng,
                           kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale, max_nb=max_nb)
    return add_multi_step(w, query_lens, rng=rng)


def _name(config: int, kv_dtype: str) -> str:
    """Workload name; an fp8- or int8-cache variant of a bf16 workload says so."""
    base = CONFIG_NAMES[config]
    return base if kv_dtype not in ("fp8", "int8") else base.replace("-bf16", "") + f"-{kv_dtype}kv"


def _config1(seed: int) -> Workload:
    # Tiny fp32 MHA: 2 sequences of 17 and 33 tokens (the new token opens a
    # fresh block in both), pool of 16 blocks, tables drawn from a permutation.
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = [17, 33]
    return scattered_workload(CONFIG_NAMES[1], "f32", B=2, H=2, H_kv=2, d=64,
                              context_lens=ctx, seed=seed, rng=rng, num_blocks=16)


def _config2(seed: int, kv_dtype: str = "bf16") -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(512, 2048, size=64, endpoint=True)
    return scattered_workload(_name(2, kv_dtype), "bf16", B=64, H=32, H_kv=32, d=128,
                              context_lens=ctx, seed=seed, rng=rng, max_nb=128,
                              kv_dtype=kv_dtype)


def _config3(seed: int, kv_dtype: str = "bf16") -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    draw = rng.lognormal(mean=math.log(1800.0), sigma=1.0, size=256)
    ctx = np.clip(np.rint(draw), 64, 8192).astype(np.int64)
    return scattered_workload(_name(3, kv_dtype), "bf16", B=256, H=64, H_kv=8, d=128,
                              context_lens=ctx, seed=seed, rng=rng, max_nb=512,
                              kv_dtype=kv_dtype)


def _config4(seed: int, kv_dtype: str = "bf16") -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = [100000, 65536, 32768, 4096, 2048, 1024, 300, 17]
    return scattered_workload(_name(4, kv_dtype), "bf16", B=8, H=32, H_kv=8, d=128,
                              context_lens=ctx, seed=seed, rng=rng, max_nb=6250,
                              partition_size=512, kv_dtype=kv_dtype)


SHARED_PREFIX_BLOCKS = 64
SHARED_PREFIX_STEPS = 50


def shared_prefix_workload(seed: int, B: int = 128, H: int = 32, H_kv: int = 8,
                           d: int = 128, steps: int = SHARED_PREFIX_STEPS,
                           prefix_blocks: int = SHARED_PREFIX_BLOCKS,
                           private_range=(16, 300), name: Optional[str] = None,
                           kv_dtype: str = "bf16") -> Workload:
    """Continuous decode over a shared prefix.

    Every sequence's table starts with the same `prefix_blocks` physical blocks,
    then private blocks for its own tokens. Each step appends one token per
    sequence; a sequence takes the next block of a seeded free list whenever its
    new token opens a block. The returned block table is the one after the last
    step; entries a step does not reach are never read by that step.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    private = rng.integers(private_range[0], private_range[1], size=B, endpoint=True)
    prefix_tokens = prefix_blocks * BLOCK_SIZE
    final_private_blocks = [_blocks_for(int(p) + steps) for p in private]
    num_blocks = prefix_blocks + int(math.ceil(1.25 * sum(final_private_blocks)))
    perm = rng.permutation(num_blocks).astype(np.int32)
    prefix = perm[:prefix_blocks]
    free = list(perm[prefix_blocks:])
    max_nb = _blocks_for(prefix_tokens + int(private.max()) + steps)
    tables = np.full((B, max_nb), TABLE_SENTINEL, dtype=np.int32)
    tables[:, :prefix_blocks] = prefix[None, :]
    for b in range(B):
        n = _blocks_for(int(private[b]))
        for j in range(n):
            tables[b, prefix_blocks + j] = free.pop(0)
    ctx_per_step = []
    for s in range(steps):
        ctx_s = np.empty(B, dtype=np.int32)
        for b in range(B):
            pos = prefix_tokens + int(private[b]) + s       # the new token's position
            if pos % BLOCK_SIZE == 0:                        # it opens a fresh block
                tables[b, pos // BLOCK_SIZE] = free.pop(0)
            ctx_s[b] = pos + 1
        ctx_per_step.append(ctx_s)
    dtype = "bf16"
    qs = [_normal_bits(rng, B * H * d, dtype).reshape(B, H, d) for _ in range(steps)]
    k_pool = kv_pool(seed, 1, num_blocks, H_kv, d, kv_dtype)
    v_pool = kv_pool(seed, 2, num_blocks, H_kv, d, kv_dtype)
    step_list = []
    for s in range(steps):
        nk = _normal_bits(rng, B * H_kv * d, dtype).reshape(B, H_kv, d)
        nv = _normal_bits(rng, B * H_kv * d, dtype).reshape(B, H_kv, d)
        step_list.append(DecodeStep(context_lens=ctx_per_step[s], q=qs[s], new_k=nk, new_v=nv))
    return Workload(name=name or _name(5, kv_dtype), dtype=dtype, B=B, H=H, H_kv=H_kv, d=d,
                    num_blocks=num_blocks, max_nb=max_nb, scale=1.0 / math.sqrt(d),
                    partition_size=0, block_tables=tables, k_pool=k_pool, v_pool=v_pool,
                    steps=step_list, seed=seed, kv_dtype=kv_dtype)


def make_workload(config: int, seed: Optional[int] = None, kv_dtype: str = "") -> Workload:
    """Build workload `config` (1..5) with its default seed (= config number).

    kv_dtype "fp8" / "int8" gives the same shapes, lengths, tables and
    activations with an fp8 cache (per-tensor scales 1.0) or an int8 cache (per
    row scales) (configs 2..5; pool bytes follow the recipes of _pool_bits and
    kv_pool).
    """
    seed = config if seed is None else seed
    if kv_dtype and kv_dtype not in ("fp8", "int8", "bf16", "f32"):
        raise ValueError(f"unsupported kv_dtype {kv_dtype!r}")
    if config == 1:
        if kv_dtype in ("fp8", "int8"):
            raise ValueError("workload 1 is float32; fp8 and int8 caches serve bf16 activations")
        return _config1(seed)
    kv = kv_dtype if kv_dtype in ("fp8", "int8") else "bf16"
    if config == 2:
        return _config2(seed, kv)
    if config == 3:
        return _config3(seed, kv)
    if config == 4:
        return _config4(seed, kv)
    if config == 5:
        return shared_prefix_workload(seed, kv_dtype=kv)
    raise ValueError(f"no workload {config}")

"""Float64 CPU oracle of decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU baseline, never by the product path.

Pages cited (titles as the pages give them):
  [FDE]  "Forward Deployed Engineering Interview", Ch.2 "Batching and the KV
         Cache": section 6 (bytes per token), section 8 (paging, the
         block_manager.py teaching model).
  [API]  "Anthropic Interview: Design an LLM Inference API with GPU Batching":
         Key concepts (Paged KV memory), 4. Data model (4.1, 4.2).
  [QA]   "MLSys Engineer - Inference Systems Q&A": Q1 (PagedAttention, the
         kernel rewrite), Q3 (pool size, layout for coalesced access), Q4
         (online softmax, fp32 accumulation).
  [WB]   "LLM inference and serving" workbook: The equations (KV-cache size,
         roofline balance point, decode throughput ceiling), Code from memory
         (naive incremental decoding, the step() function).
  [SRV]  "Ch.29 Building a Production LLM Serving Stack": 29.1.2 (block
         accounting worked example), 29.2.1 (attention intensity).
  [FDE9] "Forward Deployed Engineering Interview", Ch.2 section 9 (shrinking
         the cache: an fp8_e4m3 cache, available on ROCm, halves every row;
         scales are per tensor; windowed layers such as gpt-oss's 128-token
         band cap what a layer keeps) and the annotated serving configuration
         of the same chapter (--kv-cache-dtype fp8: every scale is 1.0 without
         calibration).
  [QA3]  same Q&A page, Q3 item 4 (local-attention layers need only the last
         W tokens) and Q4 (sliding-window attention: the first K tile a query
         at position q_pos needs starts at q_pos + 1 - W, rounded down to the
         tile; tiles wholly before it are skipped).
  [QA8]  same Q&A page, Q3 item 1 (quantise the KV cache to INT8 with one
         scale per token, the row's largest magnitude over 127; dequantise
         before the softmax).

What the oracle computes is the plain definition: decode attention over a
paged cache equals ordinary softmax attention of one query over its
sequence's de-paged, contiguous K/V ([WB] step(): append the new row, then
softmax(K q / sqrt(d)) V over all rows; [QA] Q1: the paged kernel differs from
the contiguous one only in addressing).  Nothing is blocked, fused or reordered.

Readings taken where the pages are silent (each listed in the design notes):
  * context_len counts the token written this step ([WB] step() appends before
    attending; its printed check counts prompt + decoded rows).
  * query head h reads KV head h // (H / H_kv) (contiguous groups).
  * the in-block layout of the pool (the pages fix only the block-table
    mapping; [QA] Q1's address formula omits the token and head strides) is
    the one the C ABI documents, restated here independently:
        K element (p, h, t, x) at (((p*H_kv + h)*(d/X) + x//X)*16 + t)*X + x%X
        V element (p, h, t, x) at ((p*H_kv + h)*d + x)*16 + t
    with X = 16 bytes / element size (8 for bf16, 4 for fp32, 16 for fp8).
  * ctx <= 0 gives an all-zero output (no token to attend to).
  * split-KV partitions are logical token ranges [k*P, (k+1)*P).
  * sliding window ([QA3]): with window W > 0 a query at position p attends to
    positions max(0, p - W + 1) .. p, i.e. its own position and the W - 1
    before it; W = 0 means the whole context.  In split mode the partitions of
    a windowed query start at the block holding its first visible position:
    partition k covers [r + k*P, r + (k+1)*P) with r = 16 * floor(first / 16),
    positions before `first` getting no weight.
  * fp8 cache ([FDE9]): elements are OCP E4M3 codes (the format ROCm's
    fp8_e4m3 names); a cached value is code value * per-tensor scale.  The
    write stores the nearest E4M3 value of x / scale, the division done in
    float32, ties to the even code; magnitudes beyond 448 (the largest finite
    E4M3 value; the format has no infinities) store +-448, and NaN stores
    sign | 0x7F.  Queries and outputs stay bf16.
  * int8 cache ([QA8]): one scale per (token, KV head) row of K and of V, in
    float32: s = a / 127 with a the row's largest finite magnitude (0 for a
    row with none); element code = the integer nearest x / s (float32
    division), ties to even, clamped to +-127; a non-finite element, or any
    element of a row with s = 0, stores code 0.  A cached value is code * s.
    Each cache buffer holds the codes (the fp8 layout: 16 codes per chunk)
    followed by the scales, scale (p, h, t) at byte
    codes_bytes + 4 * ((p * H_kv + h) * 16 + t).

Parity status: every function below is pinned by tests/test_oracle_pins.py
against printed page values, closed forms, library routines or invariants.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

__all__ = [
    "BLOCK",
    "bits_to_f64",
    "act_dtype",
    "chunk_elems",
    "E4M3_MAX",
    "e4m3_value",
    "e4m3_encode",
    "e4m3_quantize",
    "k_offset",
    "v_offset",
    "blocks_needed",
    "slot_mapping",
    "window_first",
    "INT8_MAX",
    "int8_quantize_rows",
    "int8_codes_bytes",
    "int8_scale_offset",
    "int8_read_scales",
    "int8_write_scales",
    "chunk_slots",
    "reshape_and_cache",
    "gather_sequence",
    "decode",
    "decode_sequence",
    "decode_multi",
    "partials",
    "reduce",
    "kv_bytes",
    "kv_bytes_per_token",
    "kv_bytes_per_token_mla",
    "ridge_intensity",
    "decode_tokens_per_s_ceiling",
    "decode_step_floor_s",
]

BLOCK = 16  # tokens per physical block ([QA] Q1: "typically 16 tokens")


# --------------------------------------------------------------------------
# element encodings
# --------------------------------------------------------------------------
def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored bit patterns to float64.

    bf16 is the top half of a float32, so shifting its 16 bits up by 16 gives
    that float32 exactly; float32 widens to float64 exactly.
    """
    bits = np.asarray(bits)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        if dtype == "bf16":
            return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        if dtype == "f32":
            return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_value(bits)
    if dtype == "int8":
        return np.asarray(bits).astype(np.uint8).view(np.int8).astype(np.float64)
    raise ValueError(dtype)


def act_dtype(dtype: str) -> str:
    """Element type of query, output and the rows handed to the cache write
    for a cache of element type `dtype` (fp8 and int8 caches serve bf16
    activations)."""
    return "bf16" if dtype in ("fp8", "int8") else dtype


def chunk_elems(dtype: str) -> int:
    """Elements per 16-byte chunk of the K layout."""
    return {"bf16": 8, "f32": 4, "fp8": 16, "int8": 16}[dtype]


# --------------------------------------------------------------------------
# fp8 (E4M3) cache elements, [FDE9]
# --------------------------------------------------------------------------
E4M3_MAX = 448.0  # largest finite E4M3 magnitude: (1 + 6/8) * 2**8


def e4m3_value(codes) -> np.ndarray:
    """Float64 value of E4M3 codes.

    The format: one sign bit, four exponent bits with bias 7, three mantissa
    bits.  Exponent field 0 is subnormal, value m/8 * 2**-6; otherwise the value
    is (1 + m/8) * 2**(e - 7).  Exponent 15 with mantissa 7 is NaN (no
    infinities), so the largest finite magnitude is 448.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of float32 values: the nearest finite E4M3 value, a tie going
    to the code whose mantissa is even; magnitudes beyond 448 give +-448; NaN
    gives sign | 0x7F; the sign of -0.0 is kept."""
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(np.abs(x), E4M3_MAX))
    table = e4m3_value(np.arange(0x7F))       # codes 0..126: 0 .. 448, increasing
    hi = np.minimum(np.searchsorted(table, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    neg = np.signbit(x)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, np.where(neg, 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def e4m3_quantize(bits: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Codes of stored activation values (bit patterns of `dtype`) under a
    per-tensor scale: e4m3_encode(x / scale), the division in float32."""
    x = bits_to_f64(bits, dtype).astype(np.float32)   # exact: bf16/f32 values
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        q = x / np.float32(scale)
    return e4m3_encode(q)


# --------------------------------------------------------------------------
# int8 cache elements with per-token scales, [QA8]
# --------------------------------------------------------------------------
INT8_MAX = 127


def int8_quantize_rows(bits: np.ndarray, dtype: str):
    """Codes (uint8 bytes of int8 values) and float32 scales of rows [..., d]
    of activation values (bit patterns of `dtype`): per row, s = a / 127 with a
    the largest finite |x| (0 if none), code = round-half-even(x / s) clamped
    to +-127, both divisions in float32; code 0 where x is not finite or s = 0."""
    x = bits_to_f64(bits, dtype).astype(np.float32)          # exact: bf16/f32 values
    finite = np.isfinite(x)
    a = np.max(np.where(finite, np.abs(x), np.float32(0)), axis=-1)
    s = (a / np.float32(INT8_MAX)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        q = (x / s[..., None]).astype(np.float32)
    ok = finite & (s[..., None] > 0)
    code = np.where(ok, np.clip(np.rint(np.where(ok, q, 0)), -INT8_MAX, INT8_MAX), 0)
    return code.astype(np.int8).view(np.uint8), s


def int8_codes_bytes(pool_len: int, d: int) -> int:
    """Bytes of the code region of an int8 cache buffer of pool_len bytes:
    each (block, head, slot) row holds d codes and one 4-byte scale."""
    return pool_len // (d + 4) * d


def int8_scale_offset(p, h, t, H_kv: int, d: int, pool_len: int):
    """Byte offset of the scale of row (block p, kv head h, slot t)."""
    p = np.asarray(p, dtype=np.int64)
    return int8_codes_bytes(pool_len, d) + 4 * ((p * H_kv + h) * BLOCK + np.asarray(t))


def int8_read_scales(pool: np.ndarray, offsets) -> np.ndarray:
    """float32 scales stored at byte offsets (little-endian)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    raw = np.stack([pool[offsets + k] for k in range(4)], axis=-1).astype(np.uint8)
    return raw.reshape(-1).view(np.float32).reshape(offsets.shape)


def int8_write_scales(pool: np.ndarray, offsets, scales) -> None:
    """Store float32 scales at byte offsets (in place)."""
    offsets = np.asarray(offsets, dtype=np.int64).reshape(-1)
    raw = np.asarray(scales, dtype=np.float32).reshape(-1).view(np.uint8).reshape(-1, 4)
    for k in range(4):
        pool[offsets + k] = raw[:, k]


# --------------------------------------------------------------------------
# the pool layout, restated from the documented formula
# --------------------------------------------------------------------------
def k_offset(p, h, t, x, H_kv: int, d: int, dtype: str):
    """Element offset of K[block p, kv head h, in-block token t, dim x]."""
    X = chunk_elems(dtype)
    p = np.asarray(p, dtype=np.int64)
    tile = (p * H_kv + h) * (d // X)
    return ((tile + np.asarray(x) // X) * BLOCK + np.asarray(t)) * X + np.asarray(x) % X


def v_offset(p, h, t, x, H_kv: int, d: int, dtype: str):
    """Element offset of V[block p, kv head h, in-block token t, dim x]."""
    p = np.asarray(p, dtype=np.int64)
    return ((p * H_kv + h) * d + np.asarray(x)) * BLOCK + np.asarray(t)


# --------------------------------------------------------------------------
# block bookkeeping arithmetic
# --------------------------------------------------------------------------
def blocks_needed(tokens: int, block_size: int = BLOCK) -> int:
    """Blocks a sequence of `tokens` tokens occupies: ceil(tokens / block).

    [SRV] 29.1.2 worked example sizes requests this way (5,000 tokens -> 313
    blocks); [QA] Q1 bounds the waste by one partial block.
    """
    return -(-int(tokens) // block_size)


def slot_mapping(block_tables: np.ndarray, context_lens: np.ndarray) -> np.ndarray:
    """Physical slot of each sequence's newest token (position ctx - 1).

    [QA] Q1: logical position i lives in block block_table[i // block_size] at
    offset i % block_size; the slot number is block * 16 + offset.  A sequence
    with ctx <= 0 has no new token: slot -1 (skipped by the cache write).
    """
    tables = np.asarray(block_tables)
    ctx = np.asarray(context_lens, dtype=np.int64)
    out = np.full(ctx.shape[0], -1, dtype=np.int64)
    for b in range(ctx.shape[0]):
        n = int(ctx[b])
        if n <= 0:
            continue
        pos = n - 1
        out[b] = int(tables[b, pos // BLOCK]) * BLOCK + pos % BLOCK
    return out


def chunk_slots(block_tables: np.ndarray, context_lens: np.ndarray,
                query_start: np.ndarray) -> np.ndarray:
    """Slots of the n_b newest tokens of each sequence (positions ctx_b - n_b ..
    ctx_b - 1), n_b = query_start[b+1] - query_start[b]: the [QA] Q1 mapping per
    position.  -1 where a position is negative (n_b > ctx_b)."""
    tables = np.asarray(block_tables)
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.full(int(qs[-1]), -1, dtype=np.int64)
    for b in range(len(context_lens)):
        n = int(qs[b + 1] - qs[b])
        for j in range(n):
            pos = int(context_lens[b]) - n + j
            if pos >= 0:
                out[qs[b] + j] = int(tables[b, pos // BLOCK]) * BLOCK + pos % BLOCK
    return out


# --------------------------------------------------------------------------
# the cache write
# --------------------------------------------------------------------------
def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray,
                      value: np.ndarray, slots: np.ndarray, H_kv: int, d: int,
                      dtype: str, num_blocks: int, k_scale: float = 1.0,
                      v_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Write each token's K and V rows into its slot; return new pools.

    [WB] step(): the cache append, K and V grow by one row per token and old
    rows are never recomputed; [FDE] section 8 append(): the token goes into the
    last block of the table.  For bf16/fp32 caches a bit copy: -0.0 and NaN
    payloads survive.  For an fp8 cache the rows are bf16 and each element is
    stored as e4m3_quantize(x, k_scale or v_scale) ([FDE9]).  A negative slot is
    skipped.  Two tokens naming one slot in one call would race on a GPU, so the
    oracle refuses them, as it refuses slots past the pool.
    """
    k_pool = np.array(k_pool, copy=True)
    v_pool = np.array(v_pool, copy=True)
    key = np.asarray(key).reshape(-1, H_kv, d)
    value = np.asarray(value).reshape(-1, H_kv, d)
    ks = vs = None
    if dtype == "fp8":
        key = e4m3_quantize(key, act_dtype(dtype), k_scale)
        value = e4m3_quantize(value, act_dtype(dtype), v_scale)
    elif dtype == "int8":
        key, ks = int8_quantize_rows(key, act_dtype(dtype))
        value, vs = int8_quantize_rows(value, act_dtype(dtype))
    slots = np.asarray(slots, dtype=np.int64)
    live = [int(s) for s in slots if s >= 0]
    if len(set(live)) != len(live):
        raise ValueError("duplicate slot in one cache write")
    for i, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        if s >= num_blocks * BLOCK:
            raise ValueError(f"slot {s} outside a pool of {num_blocks} blocks")
        blk, off = divmod(s, BLOCK)
        for h in range(H_kv):
            xs = np.arange(d)
            k_pool[k_offset(blk, h, off, xs, H_kv, d, dtype)] = key[i, h]
            v_pool[v_offset(blk, h, off, xs, H_kv, d, dtype)] = value[i, h]
            if dtype == "int8":
                int8_write_scales(k_pool, [int8_scale_offset(blk, h, off, H_kv, d, len(k_pool))],
                                  [ks[i, h]])
                int8_write_scales(v_pool, [int8_scale_offset(blk, h, off, H_kv, d, len(v_pool))],
                                  [vs[i, h]])
    return k_pool, v_pool


# --------------------------------------------------------------------------
# de-paging and attention
# --------------------------------------------------------------------------
def gather_sequence(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray,
                    ctx: int, kvh: int, H_kv: int, d: int, dtype: str,
                    k_scale: float = 1.0, v_scale: float = 1.0
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Contiguous float64 K, V [ctx, d] of one sequence and KV head.

    Token t is read from block table_row[t // 16], slot t % 16 ([QA] Q1).  Only
    the first ceil(ctx / 16) table entries and the first ctx tokens are read.
    An fp8 cache's values are code value * scale ([FDE9]; exact in float64).
    """
    t = np.arange(int(ctx), dtype=np.int64)
    if t.size == 0:
        return np.zeros((0, d)), np.zeros((0, d))
    blocks = np.asarray(table_row, dtype=np.int64)[t // BLOCK]
    xs = np.arange(d, dtype=np.int64)
    ko = k_offset(blocks[:, None], kvh, (t % BLOCK)[:, None], xs[None, :], H_kv, d, dtype)
    vo = v_offset(blocks[:, None], kvh, (t % BLOCK)[:, None], xs[None, :], H_kv, d, dtype)
    K = bits_to_f64(k_pool[ko], dtype)
    V = bits_to_f64(v_pool[vo], dtype)
    if dtype == "fp8":
        K = K * float(np.float32(k_scale))
        V = V * float(np.float32(v_scale))
    elif dtype == "int8":                    # [QA8]: code * the row's scale (exact in f64)
        K = K * int8_read_scales(k_pool, int8_scale_offset(blocks, kvh, t % BLOCK, H_kv, d,
                                                           len(k_pool))).astype(np.float64)[:, None]
        V = V * int8_read_scales(v_pool, int8_scale_offset(blocks, kvh, t % BLOCK, H_kv, d,
                                                           len(v_pool))).astype(np.float64)[:, None]
    return K, V


def window_first(pos: int, window: int) -> int:
    """First position a query at position pos sees ([QA3]): pos - W + 1, not
    below 0; 0 for W = 0 (the whole context)."""
    return max(0, int(pos) - int(window) + 1) if window > 0 else 0


def decode_sequence(k_pool, v_pool, q_b: np.ndarray, table_row, ctx: int,
                    H: int, H_kv: int, d: int, dtype: str, scale: float,
                    k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0) -> np.ndarray:
    """Output [H, d] of one sequence: softmax(scale * K q_h) V per query head.

    [WB] step(): attn = softmax(K @ q / sqrt(d)); ctx = attn @ V, over every
    cached row including the new one; with a window W > 0, over the rows of
    positions window_first(ctx - 1, W) .. ctx - 1 only ([QA3]).
    Max-subtracted softmax in float64.
    """
    g = H // H_kv
    out = np.zeros((H, d))
    if ctx <= 0:
        return out
    first = window_first(ctx - 1, window)
    q = bits_to_f64(q_b, act_dtype(dtype)).reshape(H, d)
    for kvh in range(H_kv):
        K, V = gather_sequence(k_pool, v_pool, table_row, ctx, kvh, H_kv, d, dtype,
                               k_scale, v_scale)
        K, V = K[first:], V[first:]
        for h in range(kvh * g, (kvh + 1) * g):
            s = scale * (K @ q[h])
            p = np.exp(s - s.max())
            out[h] = (p @ V) / p.sum()
    return out


def decode_multi(k_pool, v_pool, q_rows: np.ndarray, query_start, block_tables,
                 context_lens, H: int, H_kv: int, d: int, dtype: str, scale: float,
                 k_scale: float = 1.0, v_scale: float = 1.0, seqs=None,
                 window: int = 0) -> dict:
    """Attention of several new query tokens per sequence, causal within them.

    [API] (chunked prefill: a prompt enters in chunks, e.g. of 512 tokens,
    alongside decode steps), [QA] and [WB] (speculative decoding: the target
    verifies K draft tokens in one pass).  Sequence b's n_b = query_start[b+1]
    - query_start[b] query rows (q_rows [T, H, d] bits) are the tokens at
    positions ctx_b - n_b .. ctx_b - 1, whose K/V rows are already in the cache
    (context_lens count them); the token at position p attends to positions
    0..p: the [WB] step() attention with the rows appended one at a time
    (with a window W > 0: positions window_first(p, W) .. p, [QA3]).
    Returns {b: float64 [n_b, H, d]}.
    """
    g = H // H_kv
    qs = np.asarray(query_start, dtype=np.int64)
    out = {}
    for b in (range(len(context_lens)) if seqs is None else seqs):
        n = int(qs[b + 1] - qs[b])
        ctx = int(context_lens[b])
        rows = np.zeros((n, H, d))
        q = bits_to_f64(q_rows[qs[b]:qs[b + 1]], act_dtype(dtype)).reshape(n, H, d)
        for kvh in range(H_kv):
            K, V = gather_sequence(k_pool, v_pool, block_tables[b], ctx, kvh, H_kv, d, dtype,
                                   k_scale, v_scale)
            for j in range(n):
                p = ctx - n + j
                f = window_first(p, window)
                for h in range(kvh * g, (kvh + 1) * g):
                    sc = scale * (K[f:p + 1] @ q[j, h])
                    w = np.exp(sc - sc.max())
                    rows[j, h] = (w @ V[f:p + 1]) / w.sum()
        out[b] = rows
    return out


def decode(k_pool, v_pool, q: np.ndarray, block_tables: np.ndarray,
           context_lens: np.ndarray, H: int, H_kv: int, d: int, dtype: str,
           scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
           window: int = 0) -> np.ndarray:
    """Float64 decode-attention output [B, H, d] for a whole batch."""
    B = len(context_lens)
    out = np.zeros((B, H, d))
    for b in range(B):
        out[b] = decode_sequence(k_pool, v_pool, q[b], block_tables[b],
                                 int(context_lens[b]), H, H_kv, d, dtype, scale,
                                 k_scale, v_scale, window)
    return out


def partials(k_pool, v_pool, q, block_tables, context_lens, H: int, H_kv: int,
             d: int, dtype: str, scale: float, partition_size: int,
             k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0):
    """Per-partition (o, m, l) of split-KV decode.

    Partition k of a sequence covers logical tokens [r + k*P, min(r + (k+1)*P,
    ctx)), r = 0 without a window; with a window W, r is the start of the block
    holding the first visible position f = window_first(ctx - 1, W), and
    positions before f get no weight.  For a partition's scores s: m_k = max s,
    l_k = sum exp(s - m_k), and o_k = sum exp(s - m_k) v / l_k.  These are the
    running max and denominator of [QA] Q4's online softmax, taken over one
    partition.  Returns (o [B,H,Pmax,d], m [B,H,Pmax], l [B,H,Pmax], counts [B]).
    """
    P = int(partition_size)
    if P <= 0 or P % BLOCK:
        raise ValueError("partition size must be a positive multiple of 16")
    B = len(context_lens)
    g = H // H_kv
    first = [window_first(int(c) - 1, window) if int(c) > 0 else 0 for c in context_lens]
    r0 = [f // BLOCK * BLOCK for f in first]
    counts = np.array([-(-(max(int(c), 0) - r) // P) if int(c) > 0 else 0
                       for c, r in zip(context_lens, r0)], dtype=np.int64)
    Pmax = max(int(counts.max()) if B else 0, 1)
    o = np.zeros((B, H, Pmax, d))
    m = np.full((B, H, Pmax), -np.inf)
    l = np.zeros((B, H, Pmax))
    for b in range(B):
        n = int(context_lens[b])
        if n <= 0:
            continue
        qb = bits_to_f64(q[b], act_dtype(dtype)).reshape(H, d)
        for kvh in range(H_kv):
            K, V = gather_sequence(k_pool, v_pool, block_tables[b], n, kvh, H_kv, d, dtype,
                                   k_scale, v_scale)
            for h in range(kvh * g, (kvh + 1) * g):
                s = scale * (K @ qb[h])
                for k in range(int(counts[b])):
                    lo = max(r0[b] + k * P, first[b])
                    hi = min(r0[b] + (k + 1) * P, n)
                    sk = s[lo:hi]
                    mk = sk.max()
                    e = np.exp(sk - mk)
                    m[b, h, k] = mk
                    l[b, h, k] = e.sum()
                    o[b, h, k] = (e @ V[lo:hi]) / e.sum()
    return o, m, l, counts


def reduce(o: np.ndarray, m: np.ndarray, l: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Merge split partials by log-sum-exp.

    With M = max_k m_k and w_k = l_k exp(m_k - M): out = sum w_k o_k / sum w_k.
    This is [QA] Q4's rescale rule (multiply by exp(m_old - m_new) when the
    max rises) applied to whole partitions.  A sequence with no partition
    gives zeros.
    """
    B, H, _, d = o.shape
    out = np.zeros((B, H, d))
    for b in range(B):
        n = int(counts[b])
        if n == 0:
            continue
        for h in range(H):
            M = m[b, h, :n].max()
            w = l[b, h, :n] * np.exp(m[b, h, :n] - M)
            out[b, h] = (w @ o[b, h, :n]) / w.sum()
    return out


# --------------------------------------------------------------------------
# byte and roofline arithmetic
# --------------------------------------------------------------------------
def kv_bytes(L: int, H_kv: int, d: int, b: int, S: int, B: int) -> int:
    """KV-cache bytes = 2 * L * H_kv * d * b * S * B ([WB] KV-cache size)."""
    return 2 * L * H_kv * d * b * S * B


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, b: int = 2) -> int:
    """Bytes per token = 2 * L * H_kv * d_head * b ([FDE] section 6)."""
    return kv_bytes(layers, kv_heads, head_dim, b, 1, 1)


def kv_bytes_per_token_mla(r_kv: int, d_rope: int, layers: int, b: int = 2) -> int:
    """Latent-attention bytes per token = (r_kv + d_rope) * L * b ([FDE] section 6)."""
    return (r_kv + d_rope) * layers * b


def ridge_intensity(peak_flops: float, bandwidth: float) -> float:
    """I* = peak FLOP/s / peak bandwidth ([WB] roofline balance point)."""
    return peak_flops / bandwidth


def decode_tokens_per_s_ceiling(bandwidth: float, n_params: float,
                                bytes_per_weight: float) -> float:
    """tokens/s <= bandwidth / (N * bytes per weight) ([WB] decode ceiling)."""
    return bandwidth / (n_params * bytes_per_weight)


def decode_step_floor_s(bytes_per_step: float, bandwidth: float) -> float:
    """Bytes read per step divided by bandwidth ([FDE] section 1 decode floor)."""
    return bytes_per_step / bandwidth

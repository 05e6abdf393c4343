"""Shared helpers of the GPU parity tests: move a seeded workload to the GPU,
run one decode step through the C ABI, and compute the oracle's answer.

Poisoning: every slot a step must not read holds a NaN (bf16 0x7FC0, fp32
0x7FC00000, E4M3 0x7F; an int8 row gets NaN K and V row scales, its codes
stay): the tail of each sequence's last block, every block no table uses, and
the slot each step's new token is written to (so a decode that ran before the
write would read NaN).  Table entries past a sequence's blocks already hold an
index outside the pool.

A workload's pool holds w.kv_dtype elements (bf16, f32 or fp8 codes); its
queries, outputs and new rows hold w.dtype (bf16 for an fp8 pool).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from workloads import configs as W

NAN_BITS = {"bf16": np.uint16(0x7FC0), "f32": np.uint32(0x7FC00000), "fp8": np.uint8(0x7F)}
BF16_REL_L2 = 5e-3
BF16_MAX_ABS = 1e-2
F32_MAX_ABS = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)


def poison(w: W.Workload, first_unwritten: np.ndarray):
    """Copies of the pools with NaN in every slot at or past first_unwritten[b]
    of each sequence's blocks and in every block no sequence uses."""
    kp = w.k_pool.copy()
    vp = w.v_pool.copy()
    tile = w.H_kv * 16 * w.d
    used = np.zeros(w.num_blocks, dtype=bool)
    xs = np.arange(w.d)
    int8 = w.kv_dtype == "int8"
    nan = None if int8 else NAN_BITS[w.kv_dtype]
    nan_rows = []          # int8: (block, head, slot) rows whose scales become NaN

    def hide(blk, h, t):
        if int8:
            nan_rows.append((blk * w.H_kv + h) * 16 + t)
        else:
            kp[O.k_offset(blk, h, t, xs, w.H_kv, w.d, w.kv_dtype)] = nan
            vp[O.v_offset(blk, h, t, xs, w.H_kv, w.d, w.kv_dtype)] = nan

    for b in range(w.B):
        row = w.block_tables[b]
        nb_final = int(np.count_nonzero(row != W.TABLE_SENTINEL))
        used[row[:nb_final]] = True
        for pos in range(int(first_unwritten[b]), nb_final * 16):
            blk = int(row[pos // 16])
            for h in range(w.H_kv):
                hide(blk, h, pos % 16)
    unused = np.flatnonzero(~used)
    if int8:
        rows = (unused[:, None] * w.H_kv * 16 + np.arange(w.H_kv * 16)[None, :]).reshape(-1)
        rows = np.concatenate([rows, np.asarray(nan_rows, dtype=np.int64)])
        for pool in (kp, vp):
            pool[O.int8_codes_bytes(len(pool), w.d):].view(np.float32)[rows] = np.nan
        return kp, vp
    for blk in unused:
        kp[blk * tile:(blk + 1) * tile] = nan
        vp[blk * tile:(blk + 1) * tile] = nan
    return kp, vp


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """Upload a bit-pattern array without changing a bit."""
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(bits.dtype)
    arr = bits.view(view) if view is not None else bits
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Download a device tensor as bit patterns."""
    a = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return a.view(torch.int16).numpy().view(np.uint16)
    if dtype in ("fp8", "int8"):
        return a.view(torch.uint8).numpy()
    return a.view(torch.int32).numpy().view(np.uint32)


@dataclass
class DevWorkload:
    w: W.Workload
    pool: P.KVPool
    tables: torch.Tensor


def upload(w: W.Workload, k_pool: np.ndarray, v_pool: np.ndarray) -> DevWorkload:
    pool = P.KVPool(to_dev(k_pool), to_dev(v_pool), w.num_blocks, w.H_kv, w.d, w.kv_dtype,
                    w.k_scale, w.v_scale)
    tables = torch.from_numpy(w.block_tables).cuda()
    return DevWorkload(w=w, pool=pool, tables=tables)


def gpu_step(dw: DevWorkload, step: W.DecodeStep, partition_size: int = 0,
             max_context_len: Optional[int] = None, write: bool = True, fused: bool = False,
             one_launch: bool = False, window: int = 0):
    """One decode step on the GPU: slot mapping, cache write, decode (+ reduce);
    the first two as separate calls or (fused) as one kv_cache_append, or
    (one_launch) the whole step as kv_decode_step.
    Returns (slots, out) as device tensors."""
    w = dw.w
    ctx = torch.from_numpy(step.context_lens).cuda()
    q = to_dev(step.q)
    out = torch.empty_like(q)
    L = int(max(step.context_lens.max(), 1)) if max_context_len is None else max_context_len
    ws = None
    if partition_size:
        n = P.paged_attention_workspace_bytes(w.B, w.H, w.d, L, partition_size)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    if one_launch:
        slots = torch.full((w.B,), -7, dtype=torch.int64, device="cuda")
        P.kv_decode_step(dw.pool, out, q, to_dev(step.new_k), to_dev(step.new_v), dw.tables, ctx,
                         L, w.scale, partition_size, ws, slots, window=window)
        if partition_size:
            P.paged_attention_reduce(out, ws, ctx, L, partition_size, w.dtype, window=window)
        return slots, out
    if fused:
        slots = torch.full((w.B,), -7, dtype=torch.int64, device="cuda")
        P.kv_cache_append(dw.pool, to_dev(step.new_k), to_dev(step.new_v), dw.tables, ctx, slots)
    else:
        slots = P.kv_slot_mapping(dw.tables, ctx)
        if write:
            P.reshape_and_cache(dw.pool, to_dev(step.new_k), to_dev(step.new_v), slots)
    P.paged_attention_decode(dw.pool, out, q, dw.tables, ctx, L, w.scale, partition_size, ws,
                             window=window)
    if partition_size:
        P.paged_attention_reduce(out, ws, ctx, L, partition_size, w.dtype, window=window)
    return slots, out


def oracle_step(w: W.Workload, k_pool, v_pool, step: W.DecodeStep, seqs=None, window: int = 0):
    """Oracle slot mapping, cache write and decode (optionally for some sequences)."""
    slots = O.slot_mapping(w.block_tables, step.context_lens)
    kp, vp = O.reshape_and_cache(k_pool, v_pool, step.new_k, step.new_v, slots, w.H_kv, w.d,
                                 w.kv_dtype, w.num_blocks, w.k_scale, w.v_scale)
    seqs = range(w.B) if seqs is None else seqs
    ref = {b: O.decode_sequence(kp, vp, step.q[b], w.block_tables[b], int(step.context_lens[b]),
                                w.H, w.H_kv, w.d, w.kv_dtype, w.scale, w.k_scale, w.v_scale,
                                window=window)
           for b in seqs}
    return slots, kp, vp, ref


def assert_close(got_bits: np.ndarray, ref: dict, dtype: str, label: str = "",
                 amplitude: float = 1.0, per_row: bool = False):
    """Compare GPU output rows (bits [B, H, d]) with oracle rows {b: float64 [H, d]}.

    The max-abs bounds hold for unit-variance data; data drawn with a larger
    amplitude scales them by that amplitude (a bf16 ulp grows with the value).
    per_row: each (sequence, head) row's bf16 max-abs bound scales with that
    row's own magnitude, max(1, max |row|) (for caches whose weights carry a
    per-key scale rounded with them, so a row averaging few keys keeps a
    relative error of a few bf16 ulps)."""
    bs = sorted(ref)
    got = O.bits_to_f64(got_bits[bs], dtype)
    want = np.stack([ref[b] for b in bs])
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - want)
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS * amplitude, f"{label}: max-abs {err.max():.3e}"
        return err.max(), 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    assert rel <= BF16_REL_L2, f"{label}: rel-L2 {rel:.3e}"
    if per_row:
        rows_err = err.reshape(-1, err.shape[-1]).max(axis=1)
        rows_amp = np.maximum(1.0, np.abs(want).reshape(-1, err.shape[-1]).max(axis=1))
        k = int(np.argmax(rows_err / rows_amp))
        assert rows_err[k] <= BF16_MAX_ABS * amplitude * rows_amp[k], (
            f"{label}: row {k} max-abs {rows_err[k]:.3e} (row magnitude {rows_amp[k]:.2f})")
        return float(err.max()), rel
    assert err.max() <= BF16_MAX_ABS * amplitude, f"{label}: max-abs {err.max():.3e}"
    return float(err.max()), rel


def single_step_case(w: W.Workload, partition_size: int = 0, seqs=None, label: str = "",
                     amplitude: float = 1.0, fused: bool = False, per_row: bool = False,
                     one_launch: bool = False, window: int = 0):
    """Full parity check of one step: slots and pool bit-exact, outputs in tolerance."""
    step = w.steps[0]
    first_unwritten = step.context_lens.astype(np.int64) - 1
    kp0, vp0 = poison(w, np.maximum(first_unwritten, 0))
    dw = upload(w, kp0, vp0)
    log(f"[gpu] {label} B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} {w.kv_dtype} P={partition_size}"
        f"{' fused' if fused else ''}{' one-launch' if one_launch else ''}"
        f"{f' window={window}' if window else ''}")
    slots, out = gpu_step(dw, step, partition_size, fused=fused, one_launch=one_launch,
                          window=window)
    torch.cuda.synchronize()
    oslots, kp, vp, ref = oracle_step(w, kp0, vp0, step, seqs, window=window)
    np.testing.assert_array_equal(slots.cpu().numpy(), oslots, err_msg=f"{label}: slots")
    assert np.array_equal(from_dev(dw.pool.k_cache, w.kv_dtype), kp), f"{label}: K pool bits"
    assert np.array_equal(from_dev(dw.pool.v_cache, w.kv_dtype), vp), f"{label}: V pool bits"
    return assert_close(from_dev(out, w.dtype), ref, w.dtype, label, amplitude, per_row)


def scale_for(d: int) -> float:
    return 1.0 / math.sqrt(d)

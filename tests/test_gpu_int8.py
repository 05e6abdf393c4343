"""GPU parity of the int8 KV cache with per-token row scales ("MLSys Engineer -
Inference Systems Q&A", Q3 item 1).

- The quantising write is byte work, so it is checked bit for bit: codes and
  float32 row scales of reshape_and_cache and kv_cache_append equal the
  oracle's for rows of every magnitude, zero rows and rows holding infinities
  and NaNs.
- Decode reads the same codes and scales on both sides; outputs (bf16) keep
  the bf16 tolerances against the float64 oracle (rel-L2 <= 5e-3, max-abs
  <= 1e-2 times max(1, the row's largest magnitude)): vector-ALU and
  matrix-core kernels, single pass and split, with and without a sliding
  window.  Rows the step must not read have NaN scales.  The bound scales per
  row because the kernels take each key's weight p * v_scale as one bf16
  operand: a row that averages one or a few keys (outputs up to about 3 here)
  carries that rounding and the output's, together a few ulps of its own
  magnitude, not of 1.
- kv_copy_blocks copies a block's row scales with its codes.
- The multi-token calls (chunk write, causal attention) take int8 pools: their
  parity cases live with the bf16 and fp8 ones in test_gpu_multi.py and
  test_gpu_window.py; the chunk write of extreme rows is checked here.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from workloads import configs as W

from _harness import from_dev, log, poison, single_step_case, to_dev, upload

pytestmark = pytest.mark.gpu

LENS_LONG = [1, 15, 16, 17, 250, 700, 1100]


def _rows(n, H_kv, d, seed):
    """bf16 rows of mixed magnitudes; row 0 is zero, row 1 holds +-inf and a
    NaN, row 2 a single non-zero element."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, H_kv, d)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, size=(n, H_kv, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :, 3], x[1, :, 7], x[1, :, 11] = np.inf, -np.inf, np.nan
    x[2] = 0.0
    x[2, :, 5] = -3.0
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("d,H_kv", [(128, 4), (64, 2)])
@pytest.mark.parametrize("fused", [False, True])
def test_quantising_write_is_bit_exact(d, H_kv, fused):
    N = 96
    num_blocks = N // 16 + 3
    key, val = _rows(N, H_kv, d, 1), _rows(N, H_kv, d, 2)
    slots = np.random.default_rng(3).permutation(num_blocks * 16)[:N].astype(np.int64)
    nbytes = num_blocks * H_kv * 16 * (d + 4)
    kp0 = np.full(nbytes, 0x5A, dtype=np.uint8)
    vp0 = np.full(nbytes, 0xA5, dtype=np.uint8)
    pool = P.KVPool(to_dev(kp0), to_dev(vp0), num_blocks, H_kv, d, "int8")
    log(f"[gpu] int8 write d={d} H_kv={H_kv} fused={fused}")
    if fused:   # one sequence per token, a one-block table, the token at slot % 16
        tables = torch.from_numpy((slots // 16).astype(np.int32).reshape(N, 1)).cuda()
        ctx = torch.from_numpy((slots % 16 + 1).astype(np.int32)).cuda()
        got_slots = torch.empty(N, dtype=torch.int64, device="cuda")
        P.kv_cache_append(pool, to_dev(key), to_dev(val), tables, ctx, got_slots)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got_slots.cpu().numpy(), slots)
    else:
        P.reshape_and_cache(pool, to_dev(key), to_dev(val), torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
    kp, vp = O.reshape_and_cache(kp0, vp0, key, val, slots, H_kv, d, "int8", num_blocks)
    for name, got, want in (("K", from_dev(pool.k_cache, "int8"), kp),
                            ("V", from_dev(pool.v_cache, "int8"), vp)):
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{name} bytes differ at {bad[:8]}: got {got[bad[:8]]}, want {want[bad[:8]]}"


def _int8_workload(name, H, H_kv, d, lens, seed):
    return W.scattered_workload(name, "bf16", B=len(lens), H=H, H_kv=H_kv, d=d,
                                context_lens=lens, seed=seed, kv_dtype="int8")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (8, 2), (6, 2), (32, 8)])
@pytest.mark.parametrize("P_", [0, 32, 512])
def test_int8_decode_matches_oracle(d, H, H_kv, P_):
    w = _int8_workload("i8", H, H_kv, d, LENS_LONG, seed=301 + d + H)
    kind = P.kv_decode_kernel_kind(upload(w, w.k_pool, w.v_pool).pool, H)
    assert kind == (1 if H > H_kv else 0)
    single_step_case(w, P_, label=f"int8-d{d}-H{H}-Hkv{H_kv}", per_row=True)


@pytest.mark.parametrize("H,H_kv", [(4, 4), (32, 8)])
def test_int8_append_and_empty_rows(H, H_kv):
    lens = [0, 1, 15, 16, 17, 33, 250]
    w = _int8_workload("i8-append", H, H_kv, 128, lens, seed=311 + H)
    single_step_case(w, 0, label="int8-append", fused=True, per_row=True)
    single_step_case(w, 16, label="int8-append-split", fused=True, per_row=True)


@pytest.mark.parametrize("H,H_kv", [(4, 4), (16, 2)])
@pytest.mark.parametrize("window,P_", [(7, 0), (100, 0), (100, 32)])
def test_int8_windowed_decode(H, H_kv, window, P_):
    w = _int8_workload("i8-win", H, H_kv, 128, LENS_LONG, seed=321 + H)
    st = w.steps[0]
    kp0, vp0 = poison(w, np.maximum(st.context_lens.astype(np.int64) - 1, 0))
    dw = upload(w, kp0, vp0)
    ctx = torch.from_numpy(st.context_lens).cuda()
    P.kv_cache_append(dw.pool, to_dev(st.new_k), to_dev(st.new_v), dw.tables, ctx)
    q = to_dev(st.q)
    out = torch.empty_like(q)
    L = int(st.context_lens.max())
    ws = None
    if P_:
        ws = torch.empty(P.paged_attention_workspace_bytes(w.B, w.H, w.d, L, P_),
                         dtype=torch.uint8, device="cuda")
    log(f"[gpu] int8 window {window} P={P_} H={H} H_kv={H_kv}")
    P.paged_attention_decode(dw.pool, out, q, dw.tables, ctx, L, w.scale, P_, ws, window=window)
    if P_:
        P.paged_attention_reduce(out, ws, ctx, L, P_, "int8", window=window)
    torch.cuda.synchronize()
    slots = O.slot_mapping(w.block_tables, st.context_lens)
    kp, vp = O.reshape_and_cache(kp0, vp0, st.new_k, st.new_v, slots, w.H_kv, w.d, "int8",
                                 w.num_blocks)
    ref = {b: O.decode_sequence(kp, vp, st.q[b], w.block_tables[b], int(c), H, H_kv, 128, "int8",
                                w.scale, window=window) for b, c in enumerate(st.context_lens)}
    from _harness import assert_close
    assert_close(from_dev(out, "bf16"), ref, "bf16", f"int8-window{window}", per_row=True)


def test_copy_blocks_copies_codes_and_row_scales():
    H_kv, d, num_blocks = 2, 128, 12
    rng = np.random.default_rng(13)
    nbytes = num_blocks * H_kv * 16 * (d + 4)
    kp = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    vp = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    pool = P.KVPool(to_dev(kp), to_dev(vp), num_blocks, H_kv, d, "int8")
    src = np.array([3, 0, 7, -1, 5, 99, 4], dtype=np.int32)
    dst = np.array([9, 11, 1, 2, 5, 6, 10], dtype=np.int32)
    log("[gpu] int8 copy_blocks")
    P.kv_copy_blocks(pool, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    tile = H_kv * 16 * d
    codes = num_blocks * tile
    srow = H_kv * 16 * 4
    ek, ev = kp.copy(), vp.copy()
    for s, t in zip(src, dst):
        if 0 <= s < num_blocks and 0 <= t < num_blocks and s != t:
            for e, o in ((ek, kp), (ev, vp)):
                e[t * tile:(t + 1) * tile] = o[s * tile:(s + 1) * tile]
                e[codes + t * srow:codes + (t + 1) * srow] = o[codes + s * srow:codes + (s + 1) * srow]
    assert np.array_equal(from_dev(pool.k_cache, "int8"), ek)
    assert np.array_equal(from_dev(pool.v_cache, "int8"), ev)


def test_chunk_write_quantises_rows_of_every_magnitude():
    """kv_cache_append_chunk on an int8 pool: rows of magnitudes 2^-20..2^20,
    zero rows and rows holding +-inf and NaN, chunks that start and end inside
    blocks; codes and scales equal the oracle's bit for bit."""
    ctx, n = [40, 100, 7, 33], [13, 70, 7, 20]
    w = W.multi_token_workload("i8-chunk", "bf16", len(ctx), 8, 2, 128, ctx, n, seed=331,
                               kv_dtype="int8")
    m = w.multi
    T = int(m.query_start[-1])
    new_k, new_v = _rows(T, 2, 128, 4), _rows(T, 2, 128, 5)
    kp0, vp0 = poison(w, np.zeros(w.B, dtype=np.int64))
    dw = upload(w, kp0, vp0)
    log("[gpu] int8 chunk write, extreme rows")
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    P.kv_cache_append_chunk(dw.pool, to_dev(new_k), to_dev(new_v),
                            torch.from_numpy(m.query_start).cuda(), int(max(n)), dw.tables,
                            torch.from_numpy(m.context_lens).cuda(), slots)
    torch.cuda.synchronize()
    want = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    np.testing.assert_array_equal(slots.cpu().numpy(), want)
    kp, vp = O.reshape_and_cache(kp0, vp0, new_k, new_v, want, 2, 128, "int8", w.num_blocks)
    for name, got, exp in (("K", from_dev(dw.pool.k_cache, "int8"), kp),
                           ("V", from_dev(dw.pool.v_cache, "int8"), vp)):
        bad = np.flatnonzero(got != exp)
        assert bad.size == 0, f"{name} bytes differ at {bad[:8]}"

"""GPU parity of the fp8 (E4M3) KV cache ("Forward Deployed Engineering
Interview", Ch.2 section 9: an fp8_e4m3 cache with per-tensor scales).

- The quantising write is byte work, so it is checked bit for bit: every one of
  the 65,536 bf16 bit patterns (NaNs, infinities, subnormals, signed zeros
  included) goes through reshape_and_cache and kv_cache_append under several
  scales, and the pools must equal the oracle's codes.
- Decode reads the same codes on both sides; the outputs (bf16) keep the bf16
  tolerances against the float64 oracle: rel-L2 <= 5e-3, max-abs <= 1e-2.
- The invariances of the bf16 path hold bitwise here too.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from workloads import configs as W

from _harness import (from_dev, gpu_step, log, poison, single_step_case, to_dev, upload)

pytestmark = pytest.mark.gpu

LENS_LONG = [1, 15, 16, 17, 250, 700, 1100]
SCALES = [(1.0, 1.0), (0.37, 2.5), (0.125, 3.0)]


def _all_bf16_rows(H_kv, d):
    """[N, H_kv, d] bf16 rows holding each of the 65,536 bit patterns once."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n = 65536 // (H_kv * d)
    return bits.reshape(n, H_kv, d)


@pytest.mark.parametrize("k_scale,v_scale", SCALES)
@pytest.mark.parametrize("fused", [False, True])
def test_quantizing_write_of_every_bf16_pattern_is_bit_exact(k_scale, v_scale, fused):
    H_kv, d = 4, 128
    key = _all_bf16_rows(H_kv, d)
    val = key[::-1].copy()
    N = key.shape[0]                                   # 128 tokens
    num_blocks = N // 16 + 2
    slots = np.random.default_rng(7).permutation(num_blocks * 16)[:N].astype(np.int64)
    kp0 = np.full(num_blocks * H_kv * 16 * d, 0x5A, dtype=np.uint8)
    vp0 = kp0.copy()
    pool = P.KVPool(to_dev(kp0), to_dev(vp0), num_blocks, H_kv, d, "fp8", k_scale, v_scale)
    log(f"[gpu] fp8 write of all bf16 patterns: scales {k_scale}/{v_scale} fused={fused}")
    if fused:
        # one sequence per token: a single-block table, the new token at slot % 16
        tables = torch.from_numpy((slots // 16).astype(np.int32).reshape(N, 1)).cuda()
        ctx = torch.from_numpy((slots % 16 + 1).astype(np.int32)).cuda()
        got_slots = torch.empty(N, dtype=torch.int64, device="cuda")
        P.kv_cache_append(pool, to_dev(key), to_dev(val), tables, ctx, got_slots)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got_slots.cpu().numpy(), slots)
    else:
        P.reshape_and_cache(pool, to_dev(key), to_dev(val), torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
    kp, vp = O.reshape_and_cache(kp0, vp0, key, val, slots, H_kv, d, "fp8", num_blocks,
                                 k_scale=k_scale, v_scale=v_scale)
    gk = from_dev(pool.k_cache, "fp8")
    gv = from_dev(pool.v_cache, "fp8")
    bad = np.flatnonzero(gk != kp)
    assert bad.size == 0, f"K codes differ at {bad[:8]}: got {gk[bad[:8]]}, want {kp[bad[:8]]}"
    bad = np.flatnonzero(gv != vp)
    assert bad.size == 0, f"V codes differ at {bad[:8]}: got {gv[bad[:8]]}, want {vp[bad[:8]]}"


def _fp8_workload(name, H, H_kv, d, lens, seed, k_scale=0.5, v_scale=1.5):
    return W.scattered_workload(name, "bf16", B=len(lens), H=H, H_kv=H_kv, d=d,
                                context_lens=lens, seed=seed, kv_dtype="fp8",
                                k_scale=k_scale, v_scale=v_scale)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (8, 2), (16, 2), (6, 2), (32, 8), (64, 2)])
@pytest.mark.parametrize("P_", [0, 32, 512])
def test_fp8_decode_matches_oracle(d, H, H_kv, P_):
    w = _fp8_workload("fp8", H, H_kv, d, LENS_LONG, seed=201 + d + H)
    kind = P.kv_decode_kernel_kind(upload(w, w.k_pool, w.v_pool).pool, H)
    assert kind == (1 if H > H_kv else 0)
    single_step_case(w, P_, label=f"fp8-d{d}-H{H}-Hkv{H_kv}")


@pytest.mark.parametrize("k_scale,v_scale", SCALES)
@pytest.mark.parametrize("H,H_kv", [(4, 4), (32, 8)])
def test_fp8_scales(k_scale, v_scale, H, H_kv):
    w = _fp8_workload("fp8-scales", H, H_kv, 128, LENS_LONG, seed=231, k_scale=k_scale,
                      v_scale=v_scale)
    single_step_case(w, 0, label=f"fp8-scales-{k_scale}-{v_scale}")
    single_step_case(w, 512, label=f"fp8-scales-{k_scale}-{v_scale}-split")


@pytest.mark.parametrize("d,H,H_kv", [(128, 4, 4), (64, 4, 4), (128, 16, 2), (128, 32, 8)])
@pytest.mark.parametrize("P_", [0, 512])
def test_fp8_append_then_decode_matches_oracle(d, H, H_kv, P_):
    lens = [1, 15, 16, 17, 33, 250, 700]
    w = _fp8_workload("fp8-append", H, H_kv, d, lens, seed=241 + d + H)
    single_step_case(w, P_, label=f"fp8-append-d{d}-H{H}", fused=True)


def test_fp8_empty_and_ragged_batch():
    lens = [0, 20, 0, 33, 1]
    w = _fp8_workload("fp8-empty", 8, 2, 128, lens, seed=251)
    single_step_case(w, 0, label="fp8-empty")
    single_step_case(w, 16, label="fp8-empty-split")


def _outputs(w, kp, vp, P_=0):
    dw = upload(w, kp, vp)
    _, out = gpu_step(dw, w.steps[0], P_, write=False)
    return from_dev(out, w.dtype)


@pytest.mark.parametrize("H,H_kv", [(4, 4), (16, 2)])
def test_fp8_block_permutation_is_bitwise_invariant(H, H_kv):
    w = _fp8_workload("fp8-perm", H, H_kv, 128, LENS_LONG, seed=261)
    kp, vp = poison(w, w.steps[0].context_lens.astype(np.int64))
    base = _outputs(w, kp, vp)
    pi = np.random.default_rng(9).permutation(w.num_blocks)
    tile = w.H_kv * 16 * w.d
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    for p in range(w.num_blocks):
        kp2[pi[p] * tile:(pi[p] + 1) * tile] = kp[p * tile:(p + 1) * tile]
        vp2[pi[p] * tile:(pi[p] + 1) * tile] = vp[p * tile:(p + 1) * tile]
    used = w.block_tables != W.TABLE_SENTINEL
    w.block_tables[used] = pi[w.block_tables[used]]
    np.testing.assert_array_equal(base, _outputs(w, kp2, vp2))


@pytest.mark.parametrize("H,H_kv", [(4, 4), (16, 2)])
def test_fp8_single_token_returns_its_dequantized_value_row(H, H_kv):
    """ctx = 1 with v_scale 1: the output is the written token's E4M3 value,
    which bf16 holds exactly."""
    w = _fp8_workload("fp8-one", H, H_kv, 128, [1, 1, 1], seed=271, k_scale=0.5, v_scale=1.0)
    step = w.steps[0]
    kp, vp = poison(w, np.zeros(3, np.int64))
    dw = upload(w, kp, vp)
    _, out = gpu_step(dw, step, 0)
    got = from_dev(out, "bf16")
    want = W.f32_to_bf16_bits(
        O.e4m3_value(O.e4m3_quantize(step.new_v, "bf16", 1.0)).astype(np.float32))
    g = H // H_kv
    for b in range(3):
        for h in range(H):
            np.testing.assert_array_equal(got[b, h], want[b, h // g])

"""Pins of the oracle's fp8 (E4M3) cache: codec, quantising write, dequantising
gather.  CPU only.

The pages ask for an fp8_e4m3 cache with per-tensor scales, 1.0 when
uncalibrated ("Forward Deployed Engineering Interview", Ch.2 section 9 and the
annotated serving configuration).  The codec is pinned against torch's
float8_e4m3fn (a library routine) where the two definitions coincide, against a
brute-force nearest search, and against closed forms of the format; the
saturating overflow and the NaN rule are the oracle's stated reading.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from workloads import configs as W

ALL_BF16 = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def _torch_value(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.double().numpy()


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


# ---------------------------------------------------------------- the format
def test_e4m3_table_matches_torch_for_every_code():
    codes = np.arange(256)
    assert _same(O.e4m3_value(codes), _torch_value(codes))


def test_e4m3_format_landmarks():
    v = O.e4m3_value
    assert v(0x01) == 2.0 ** -9           # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9       # largest subnormal
    assert v(0x08) == 2.0 ** -6           # smallest normal
    assert v(0x38) == 1.0                 # exponent field 7 = bias
    assert v(0x7E) == O.E4M3_MAX == 448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x80) == 0.0 and np.signbit(v(0x80))
    assert v(0xFE) == -448.0
    finite = O.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(finite) > 0)    # codes 0..126 increase strictly


def test_e4m3_encode_matches_torch_where_both_are_defined():
    # torch rounds to nearest, ties to even, and turns |x| >= 480 into NaN; at
    # |x| <= 464 (every value that rounds to a finite code) the two agree.
    x = ALL_BF16
    inr = (np.abs(x) <= 464) & ~np.isnan(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x)
    assert inr.sum() > 30000
    np.testing.assert_array_equal(got[inr], ref[inr])


def _brute_force(x):
    """Nearest finite code by exhaustive distance, ties to the even code."""
    table = O.e4m3_value(np.arange(0x7F))
    out = []
    for v in np.asarray(x, dtype=np.float64):
        a = min(abs(v), 448.0)
        dist = np.abs(table - a)
        best = np.flatnonzero(dist == dist.min())
        code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
        out.append(code | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-12, 9.2, 3000))
    x = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    table = O.e4m3_value(np.arange(0x7F))
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)   # exact ties in float32
    x = np.concatenate([x, mids, -mids, table.astype(np.float32)])
    np.testing.assert_array_equal(O.e4m3_encode(x), _brute_force(x))


def test_e4m3_saturation_nan_and_signed_zero():
    x = np.array([448.0, 448.5, 470.0, 1e6, np.inf, -470.0, -np.inf, np.nan, -np.nan,
                  0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -10], dtype=np.float32)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF,
            0x00, 0x80, 0x00, 0x80, 0x02]
    assert O.e4m3_encode(x).tolist() == want


def test_e4m3_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_value(codes).astype(np.float32)), codes)


# ---------------------------------------------------------------- the scale
def test_quantize_with_power_of_two_scale_is_an_exact_rescaling():
    bits = (ALL_BF16.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    x = ALL_BF16
    for k in (-3, 0, 2):
        got = O.e4m3_quantize(bits, "bf16", 2.0 ** k)
        with np.errstate(over="ignore", invalid="ignore"):
            want = O.e4m3_encode((x.astype(np.float64) * 2.0 ** -k).astype(np.float32))
        np.testing.assert_array_equal(got, want)


def test_quantize_error_is_within_the_format_bound():
    # |value * s - x| <= half a unit in the last place of the code: 2**-4 |x|
    # for normal values, 2**-10 * s below the normal range.
    rng = np.random.default_rng(1)
    s = 0.37
    x32 = rng.standard_normal(20000).astype(np.float32) * np.float32(40)
    bits = W.f32_to_bf16_bits(x32)
    x = O.bits_to_f64(bits, "bf16")
    got = O.e4m3_value(O.e4m3_quantize(bits, "bf16", s)) * float(np.float32(s))
    inr = np.abs(x) / s <= 448
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(np.abs(got - x)[inr] <= bound[inr])
    assert np.all(np.abs(got[~inr]) == 448 * float(np.float32(s)))


# ---------------------------------------------------------------- cache write
def test_fp8_cache_write_quantizes_each_row_into_its_slot():
    rng = np.random.default_rng(2)
    H_kv, d, num_blocks = 2, 64, 5
    n = num_blocks * H_kv * 16 * d
    kp = np.full(n, 0x7F, dtype=np.uint8)
    vp = kp.copy()
    key = W.f32_to_bf16_bits(rng.standard_normal((3, H_kv, d)).astype(np.float32) * 3)
    val = W.f32_to_bf16_bits(rng.standard_normal((3, H_kv, d)).astype(np.float32) * 3)
    slots = np.array([5, -1, 4 * 16 + 15], dtype=np.int64)
    k2, v2 = O.reshape_and_cache(kp, vp, key, val, slots, H_kv, d, "fp8", num_blocks,
                                 k_scale=0.5, v_scale=2.0)
    qk = O.e4m3_quantize(key, "bf16", 0.5)
    qv = O.e4m3_quantize(val, "bf16", 2.0)
    changed = 0
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), 16)
        for h in range(H_kv):
            xs = np.arange(d)
            np.testing.assert_array_equal(k2[O.k_offset(blk, h, off, xs, H_kv, d, "fp8")], qk[i, h])
            np.testing.assert_array_equal(v2[O.v_offset(blk, h, off, xs, H_kv, d, "fp8")], qv[i, h])
        changed += 1
    # bytes that differ from the NaN fill: exactly 2 * H_kv * d per written token
    # (the KV-cache size formula with L = 1 and b = 1 byte per element)
    written = int(np.sum(k2 != kp)) + int(np.sum(v2 != vp))
    assert written == changed * O.kv_bytes(1, H_kv, d, 1, 1, 1)


# ---------------------------------------------------------------- decode
def _fp8_paged(seed, B, H, H_kv, d, lens, k_scale, v_scale):
    """Sequences of bf16 rows written into an fp8 pool through the oracle's
    append history; also returns the float64 dequantized rows, decoded by
    torch's float8_e4m3fn rather than the oracle's table."""
    rng = np.random.default_rng(seed)
    seq_k = [W.f32_to_bf16_bits(rng.standard_normal((n, H_kv, d)).astype(np.float32)) for n in lens]
    seq_v = [W.f32_to_bf16_bits(rng.standard_normal((n, H_kv, d)).astype(np.float32)) for n in lens]
    nb = [O.blocks_needed(n) for n in lens]
    num_blocks = sum(nb) + 2
    perm = rng.permutation(num_blocks)
    tables = np.full((B, max(max(nb), 1)), W.TABLE_SENTINEL, dtype=np.int32)
    pos = 0
    for b in range(B):
        tables[b, :nb[b]] = perm[pos:pos + nb[b]]
        pos += nb[b]
    q = W.f32_to_bf16_bits(rng.standard_normal((B, H, d)).astype(np.float32))
    kp = np.full(num_blocks * H_kv * 16 * d, 0x7F, dtype=np.uint8)
    vp = kp.copy()
    for p in range(max(lens)):
        ctx = np.array([p + 1 if p < lens[b] else 0 for b in range(B)], dtype=np.int32)
        slots = O.slot_mapping(tables, ctx)
        key = np.stack([seq_k[b][p] if p < lens[b] else np.zeros((H_kv, d), np.uint16) for b in range(B)])
        val = np.stack([seq_v[b][p] if p < lens[b] else np.zeros((H_kv, d), np.uint16) for b in range(B)])
        kp, vp = O.reshape_and_cache(kp, vp, key, val, slots, H_kv, d, "fp8", num_blocks,
                                     k_scale=k_scale, v_scale=v_scale)
    deq_k = [_torch_value(O.e4m3_quantize(k, "bf16", k_scale)) * float(np.float32(k_scale)) for k in seq_k]
    deq_v = [_torch_value(O.e4m3_quantize(v, "bf16", v_scale)) * float(np.float32(v_scale)) for v in seq_v]
    return dict(kp=kp, vp=vp, tables=tables, q=q, ctx=np.array(lens, np.int32),
                deq_k=deq_k, deq_v=deq_v)


def _sdpa(deq_k, deq_v, q, H, H_kv, d, scale):
    g = H // H_kv
    outs = []
    for b in range(len(deq_k)):
        K = torch.from_numpy(deq_k[b]).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
        V = torch.from_numpy(deq_v[b]).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
        Q = torch.from_numpy(O.bits_to_f64(q[b], "bf16")).reshape(H, 1, d)
        outs.append(torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
                    .reshape(H, d).numpy())
    return np.stack(outs)


@pytest.mark.parametrize("H,H_kv,d,lens,ks,vs", [
    (2, 2, 64, [17, 33], 1.0, 1.0),
    (8, 2, 128, [1, 16, 40], 0.5, 1.5),
    (4, 1, 64, [31, 5], 0.37, 2.2),
])
def test_fp8_decode_equals_sdpa_over_the_dequantized_rows(H, H_kv, d, lens, ks, vs):
    r = _fp8_paged(3, len(lens), H, H_kv, d, lens, ks, vs)
    scale = 1 / np.sqrt(d)
    got = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], H, H_kv, d, "fp8", scale,
                   k_scale=ks, v_scale=vs)
    ref = _sdpa(r["deq_k"], r["deq_v"], r["q"], H, H_kv, d, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    o, m, l, counts = O.partials(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], H, H_kv, d,
                                 "fp8", scale, 16, k_scale=ks, v_scale=vs)
    np.testing.assert_allclose(O.reduce(o, m, l, counts), ref, rtol=1e-12, atol=1e-13)


def test_fp8_layout_is_a_bijection_with_16_element_chunks():
    H_kv, d = 2, 128
    t = np.arange(16)[:, None]
    x = np.arange(d)[None, :]
    for h in range(H_kv):
        ko = O.k_offset(3, h, t, x, H_kv, d, "fp8")
        base = (3 * H_kv + h) * 16 * d
        assert sorted((ko - base).ravel().tolist()) == list(range(16 * d))
        # one token's 16 consecutive dims are 16 consecutive bytes
        assert np.all(np.diff(ko[5, 32:48]) == 1)


def test_fp8_planted_mistakes_are_caught(monkeypatch):
    r = _fp8_paged(4, 2, 4, 2, 64, [20, 9], 0.5, 1.5)
    scale = 0.125
    ref = _sdpa(r["deq_k"], r["deq_v"], r["q"], 4, 2, 64, scale)

    def run(ks=0.5, vs=1.5):
        return O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 4, 2, 64, "fp8", scale,
                        k_scale=ks, v_scale=vs)

    np.testing.assert_allclose(run(), ref, rtol=1e-12, atol=1e-13)
    # (1) a dropped value scale, (2) a dropped key scale
    assert not np.allclose(run(vs=1.0), ref, rtol=1e-6)
    assert not np.allclose(run(ks=1.0), ref, rtol=1e-6)
    # (3) a quantiser that multiplies by the scale instead of dividing
    real = O.pagedkv_oracle.e4m3_quantize
    wrong = lambda bits, dt, s: real(bits, dt, 1.0 / s)  # noqa: E731
    monkeypatch.setattr(O.pagedkv_oracle, "e4m3_quantize", wrong)
    monkeypatch.setattr(O, "e4m3_quantize", wrong)
    with pytest.raises(AssertionError):
        test_quantize_with_power_of_two_scale_is_an_exact_rescaling()
    monkeypatch.setattr(O.pagedkv_oracle, "e4m3_quantize", real)
    monkeypatch.setattr(O, "e4m3_quantize", real)
    # (4) an encoder that truncates instead of rounding to nearest
    real_enc = O.pagedkv_oracle.e4m3_encode

    def trunc(x):
        x = np.asarray(x, np.float32).astype(np.float64)
        table = O.e4m3_value(np.arange(0x7F))
        a = np.minimum(np.abs(x), 448.0)
        c = np.searchsorted(table, a, side="right") - 1
        return (c | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    monkeypatch.setattr(O.pagedkv_oracle, "e4m3_encode", trunc)
    x = np.float32([0.3, 1.1, -7.7, 100.0])
    assert not np.array_equal(O.pagedkv_oracle.e4m3_encode(x), _brute_force(x))
    monkeypatch.setattr(O.pagedkv_oracle, "e4m3_encode", real_enc)

"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests needs a GPU.  Each one checks the oracle against something
other than itself: values the pages print (tests/golden/page_values.json),
a library routine (torch's scaled_dot_product_attention, scipy's softmax),
closed forms, brute force on tiny inputs, and invariants the pages state.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from workloads import configs as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- page values
def test_kv_bytes_page_values(golden):
    for e in golden["kv_bytes"]:
        got = O.kv_bytes(**e["args"])
        if e["kind"] == "exact":
            assert got == e["expected"], e["cite"]
        else:
            assert abs(got - e["expected"]) <= e["rel_tol"] * e["expected"], e["cite"]


def test_kv_bytes_per_token_gib_at_128k(golden):
    for e in golden["kv_bytes_per_token_gib_128k"]:
        assert round(e["per_token"] * 131072 / 2**30, 2) == pytest.approx(e["expected"]), e["cite"]


def test_kv_bytes_mla_page_values(golden):
    for e in golden["kv_bytes_mla"]:
        assert O.kv_bytes_per_token_mla(**e["args"]) == e["expected"], e["cite"]


def test_kv_bytes_per_token_matches_formula_at_s1(golden):
    assert O.kv_bytes_per_token(80, 8, 128, 2) == 327680


def test_block_counts_page_values(golden):
    for e in golden["blocks"]:
        assert O.blocks_needed(e["tokens"]) == e["expected"], e["cite"]
    for e in golden["block_capacity"]:
        free = e["pool_blocks"] - O.blocks_needed(e["shared_tokens"]) if e["shared_tokens"] else e["pool_blocks"]
        assert free // O.blocks_needed(e["per_request_tokens"]) == e["expected"], e["cite"]


def test_internal_fragmentation_bounded_by_one_block():
    # MLSys Q&A, Q1: at most 15 unused slots per sequence.
    for n in range(1, 200):
        assert 0 <= O.blocks_needed(n) * 16 - n <= 15


def test_roofline_page_values(golden):
    for e in golden["roofline"]:
        got = getattr(O, e["fn"])(*e["args"])
        assert got == pytest.approx(e["expected"], rel=e["rel_tol"]), e["cite"]


# ---------------------------------------------------------------- layout
@pytest.mark.parametrize("dtype,H_kv,d", [("bf16", 2, 128), ("f32", 3, 64), ("bf16", 1, 64)])
def test_layout_is_a_bijection_with_contiguous_tiles(dtype, H_kv, d):
    nblk = 3
    p, h, t, x = np.meshgrid(np.arange(nblk), np.arange(H_kv), np.arange(16), np.arange(d),
                             indexing="ij")
    for fn in (O.k_offset, O.v_offset):
        off = fn(p, h, t, x, H_kv, d, dtype)
        flat = np.sort(off.ravel())
        assert np.array_equal(flat, np.arange(nblk * H_kv * 16 * d)), fn.__name__
        # every (block, head) tile is one contiguous run of 16*d elements
        base = (p * H_kv + h) * 16 * d
        assert np.all((off >= base) & (off < base + 16 * d))


def test_layout_chunk_structure():
    # K: 16-byte chunks of a token are contiguous, and for one chunk index the 16
    # tokens of a block follow one another.  V: the 16 tokens of one dim are
    # contiguous.  These are the properties the kernels' loads rely on.
    for dtype, X in (("bf16", 8), ("f32", 4)):
        H_kv, d = 2, 128
        k = O.k_offset(1, 1, 5, np.arange(X), H_kv, d, dtype)
        assert np.array_equal(np.diff(k), np.ones(X - 1))
        k_tok = O.k_offset(1, 1, np.arange(16), 0, H_kv, d, dtype)
        assert np.array_equal(np.diff(k_tok), np.full(15, X))
        v_tok = O.v_offset(1, 1, np.arange(16), 7, H_kv, d, dtype)
        assert np.array_equal(np.diff(v_tok), np.ones(15))


# ---------------------------------------------------------------- helpers
def _bf16(rng, shape):
    return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _f32(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).view(np.uint32)


def _prefill_pool(seq_k, seq_v, tables, H_kv, d, dtype, num_blocks):
    """Fill a NaN pool by replaying the append history token by token.

    seq_k[b] is [n_b, H_kv, d] bits.  Each step appends one token per live
    sequence, through the oracle's slot mapping and cache write."""
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.uint32(0x7FC00000)
    n_elem = num_blocks * H_kv * 16 * d
    kp = np.full(n_elem, nan, dtype=W.bits_dtype(dtype))
    vp = kp.copy()
    B = len(seq_k)
    lens = [s.shape[0] for s in seq_k]
    for pos in range(max(lens)):
        ctx = np.array([pos + 1 if pos < lens[b] else 0 for b in range(B)], dtype=np.int32)
        slots = O.slot_mapping(tables, ctx)
        key = np.stack([seq_k[b][pos] if pos < lens[b] else np.zeros((H_kv, d), kp.dtype)
                        for b in range(B)])
        val = np.stack([seq_v[b][pos] if pos < lens[b] else np.zeros((H_kv, d), kp.dtype)
                        for b in range(B)])
        kp, vp = O.reshape_and_cache(kp, vp, key, val, slots, H_kv, d, dtype, num_blocks)
    return kp, vp


def _random_paged(seed, B, H, H_kv, d, dtype, lens, extra_blocks=3):
    rng = np.random.default_rng(seed)
    mk = _bf16 if dtype == "bf16" else _f32
    seq_k = [mk(rng, (n, H_kv, d)) for n in lens]
    seq_v = [mk(rng, (n, H_kv, d)) for n in lens]
    nb = [O.blocks_needed(n) for n in lens]
    num_blocks = sum(nb) + extra_blocks
    perm = rng.permutation(num_blocks)
    tables = np.full((B, max(max(nb), 1)), W.TABLE_SENTINEL, dtype=np.int32)
    pos = 0
    for b in range(B):
        tables[b, :nb[b]] = perm[pos:pos + nb[b]]
        pos += nb[b]
    q = mk(rng, (B, H, d))
    kp, vp = _prefill_pool(seq_k, seq_v, tables, H_kv, d, dtype, num_blocks)
    return dict(seq_k=seq_k, seq_v=seq_v, tables=tables, q=q, kp=kp, vp=vp,
                num_blocks=num_blocks, ctx=np.array(lens, dtype=np.int32))


def _sdpa_reference(seq_k, seq_v, q, H, H_kv, d, dtype, scale):
    """torch's float64 scaled_dot_product_attention over contiguous K/V."""
    g = H // H_kv
    outs = []
    for b in range(len(seq_k)):
        K = torch.from_numpy(O.bits_to_f64(seq_k[b], dtype)).permute(1, 0, 2)  # [H_kv, n, d]
        V = torch.from_numpy(O.bits_to_f64(seq_v[b], dtype)).permute(1, 0, 2)
        K = K.repeat_interleave(g, dim=0).contiguous()
        V = V.repeat_interleave(g, dim=0).contiguous()
        Q = torch.from_numpy(O.bits_to_f64(q[b], dtype)).reshape(H, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        outs.append(o.reshape(H, d).numpy())
    return np.stack(outs)


# ---------------------------------------------------------------- attention pins
@pytest.mark.parametrize("dtype,H,H_kv,d,lens", [
    ("f32", 2, 2, 64, [17, 33]),
    ("bf16", 4, 2, 128, [1, 16, 31, 50]),
    ("bf16", 8, 1, 64, [5, 40]),
    ("f32", 6, 3, 64, [16, 64, 3]),
])
def test_paged_decode_equals_contiguous_sdpa(dtype, H, H_kv, d, lens):
    """Paged output == torch SDPA over the appended contiguous rows (fp64)."""
    r = _random_paged(11, len(lens), H, H_kv, d, dtype, lens)
    scale = 1.0 / math.sqrt(d)
    got = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], H, H_kv, d, dtype, scale)
    ref = _sdpa_reference(r["seq_k"], r["seq_v"], r["q"], H, H_kv, d, dtype, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_decode_matches_unstabilised_and_scipy_softmax():
    """Tiny inputs: direct exp(s)/sum(exp(s)) and scipy's softmax agree."""
    r = _random_paged(3, 2, 2, 2, 64, "f32", [17, 33])
    scale = 0.125
    got = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 2, 2, 64, "f32", scale)
    for b in range(2):
        for h in range(2):
            K = O.bits_to_f64(r["seq_k"][b][:, h], "f32")
            V = O.bits_to_f64(r["seq_v"][b][:, h], "f32")
            q = O.bits_to_f64(r["q"][b, h], "f32")
            s = scale * np.einsum("nd,d->n", K, q)
            e = np.exp(s)                           # no max subtraction: fine at this size
            np.testing.assert_allclose(got[b, h], (e / e.sum()) @ V, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(got[b, h], scipy.special.softmax(s) @ V,
                                       rtol=1e-12, atol=1e-14)


def test_prefill_history_reproduces_the_rows():
    """Gathering a sequence returns exactly the appended rows, in order."""
    r = _random_paged(5, 3, 4, 2, 128, "bf16", [1, 16, 47])
    for b in range(3):
        for h in range(2):
            K, V = O.gather_sequence(r["kp"], r["vp"], r["tables"][b], int(r["ctx"][b]), h,
                                     2, 128, "bf16")
            np.testing.assert_array_equal(K, O.bits_to_f64(r["seq_k"][b][:, h], "bf16"))
            np.testing.assert_array_equal(V, O.bits_to_f64(r["seq_v"][b][:, h], "bf16"))


def test_new_token_opens_fresh_block_and_count_includes_it():
    """The workbook's step() attends over prompt + decoded rows; with ctx 17 the
    newest token sits in slot 0 of the sequence's second block."""
    tables = np.array([[5, 9, W.TABLE_SENTINEL]], dtype=np.int32)
    assert O.slot_mapping(tables, np.array([17]))[0] == 9 * 16 + 0
    assert O.slot_mapping(tables, np.array([16]))[0] == 5 * 16 + 15
    assert O.slot_mapping(tables, np.array([33]))[0] == int(W.TABLE_SENTINEL) * 16 + 0
    assert O.slot_mapping(tables, np.array([0]))[0] == -1


def test_block_permutation_invariance():
    """Relabelling physical blocks (moving the data) leaves the output unchanged."""
    r = _random_paged(7, 3, 4, 2, 64, "bf16", [20, 33, 48], extra_blocks=5)
    H, H_kv, d = 4, 2, 64
    base = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], H, H_kv, d, "bf16", 0.125)
    pi = np.random.default_rng(1).permutation(r["num_blocks"])
    tile = H_kv * 16 * d
    kp2 = np.empty_like(r["kp"])
    vp2 = np.empty_like(r["vp"])
    for p in range(r["num_blocks"]):
        kp2[pi[p] * tile:(pi[p] + 1) * tile] = r["kp"][p * tile:(p + 1) * tile]
        vp2[pi[p] * tile:(pi[p] + 1) * tile] = r["vp"][p * tile:(p + 1) * tile]
    t2 = r["tables"].copy()
    used = t2 != W.TABLE_SENTINEL
    t2[used] = pi[t2[used]]
    moved = O.decode(kp2, vp2, r["q"], t2, r["ctx"], H, H_kv, d, "bf16", 0.125)
    np.testing.assert_array_equal(base, moved)


def test_shared_prefix_equals_private_copies():
    """Sequences pointing at the same prefix blocks == the same sequences with copies."""
    rng = np.random.default_rng(9)
    H, H_kv, d, dtype = 4, 2, 64, "bf16"
    tile = H_kv * 16 * d
    n_prefix, B = 3, 4
    tails = [5, 16, 17, 30]
    nb_tail = [O.blocks_needed(t) for t in tails]
    nblk_shared = n_prefix + sum(nb_tail)
    nblk_private = B * n_prefix + sum(nb_tail)
    kp_s = _bf16(rng, nblk_shared * tile)
    vp_s = _bf16(rng, nblk_shared * tile)
    maxnb = n_prefix + max(nb_tail)
    t_s = np.full((B, maxnb), W.TABLE_SENTINEL, dtype=np.int32)
    t_p = t_s.copy()
    kp_p = np.empty(nblk_private * tile, dtype=np.uint16)
    vp_p = np.empty_like(kp_p)
    nxt_s, nxt_p = n_prefix, 0
    for b in range(B):
        t_s[b, :n_prefix] = np.arange(n_prefix)
        for j in range(n_prefix):
            kp_p[nxt_p * tile:(nxt_p + 1) * tile] = kp_s[j * tile:(j + 1) * tile]
            vp_p[nxt_p * tile:(nxt_p + 1) * tile] = vp_s[j * tile:(j + 1) * tile]
            t_p[b, j] = nxt_p
            nxt_p += 1
        for j in range(nb_tail[b]):
            src = nxt_s
            t_s[b, n_prefix + j] = src
            kp_p[nxt_p * tile:(nxt_p + 1) * tile] = kp_s[src * tile:(src + 1) * tile]
            vp_p[nxt_p * tile:(nxt_p + 1) * tile] = vp_s[src * tile:(src + 1) * tile]
            t_p[b, n_prefix + j] = nxt_p
            nxt_s += 1
            nxt_p += 1
    ctx = np.array([n_prefix * 16 + t for t in tails], dtype=np.int32)
    q = _bf16(rng, (B, H, d))
    a = O.decode(kp_s, vp_s, q, t_s, ctx, H, H_kv, d, dtype, 0.125)
    b_ = O.decode(kp_p, vp_p, q, t_p, ctx, H, H_kv, d, dtype, 0.125)
    np.testing.assert_array_equal(a, b_)


# ---------------------------------------------------------------- closed forms
def test_single_token_returns_its_value_row():
    r = _random_paged(2, 2, 2, 2, 64, "f32", [1, 1])
    got = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 2, 2, 64, "f32", 0.125)
    for b in range(2):
        np.testing.assert_array_equal(got[b], O.bits_to_f64(r["seq_v"][b][0], "f32"))


def test_zero_query_and_identical_keys_give_mean_of_values():
    r = _random_paged(4, 2, 2, 2, 64, "f32", [7, 40])
    zero_q = np.zeros_like(r["q"])
    got = O.decode(r["kp"], r["vp"], zero_q, r["tables"], r["ctx"], 2, 2, 64, "f32", 0.125)
    for b in range(2):
        for h in range(2):
            mean = O.bits_to_f64(r["seq_v"][b][:, h], "f32").mean(axis=0)
            np.testing.assert_allclose(got[b, h], mean, rtol=1e-12, atol=1e-14)
    # identical key rows: all scores equal, so the mean again
    same_k = [np.repeat(s[:1], s.shape[0], axis=0) for s in r["seq_k"]]
    kp, vp = _prefill_pool(same_k, r["seq_v"], r["tables"], 2, 64, "f32", r["num_blocks"])
    got = O.decode(kp, vp, r["q"], r["tables"], r["ctx"], 2, 2, 64, "f32", 0.125)
    for b in range(2):
        for h in range(2):
            mean = O.bits_to_f64(r["seq_v"][b][:, h], "f32").mean(axis=0)
            np.testing.assert_allclose(got[b, h], mean, rtol=1e-12, atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(12)
    n, d = 21, 64
    q = rng.standard_normal(d).astype(np.float32)
    K = rng.standard_normal((n, 1, d)).astype(np.float32)
    j = 13
    K[j, 0] = 40.0 * q                               # score ~ 40^2 * |q|^2 / 8: dominates
    V = rng.standard_normal((n, 1, d)).astype(np.float32)
    tables = np.array([[2, 0]], dtype=np.int32)
    kp, vp = _prefill_pool([K.view(np.uint32)], [V.view(np.uint32)], tables, 1, d, "f32", 3)
    got = O.decode(kp, vp, q.view(np.uint32).reshape(1, 1, d), tables, np.array([n]), 1, 1, d,
                   "f32", 0.125)
    np.testing.assert_allclose(got[0, 0], V[j, 0].astype(np.float64), rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    H, H_kv, d = 8, 2, 64
    g = H // H_kv
    r = _random_paged(6, 2, H, H_kv, d, "bf16", [19, 36])
    gqa = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], H, H_kv, d, "bf16", 0.125)
    rep_k = [np.repeat(s, g, axis=1) for s in r["seq_k"]]
    rep_v = [np.repeat(s, g, axis=1) for s in r["seq_v"]]
    kp, vp = _prefill_pool(rep_k, rep_v, r["tables"], H, d, "bf16", r["num_blocks"])
    mha = O.decode(kp, vp, r["q"], r["tables"], r["ctx"], H, H, d, "bf16", 0.125)
    np.testing.assert_array_equal(gqa, mha)


def test_empty_context_gives_zero():
    r = _random_paged(8, 2, 2, 2, 64, "f32", [0, 5])
    got = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 2, 2, 64, "f32", 0.125)
    assert np.all(got[0] == 0.0)


# ---------------------------------------------------------------- split / reduce
@pytest.mark.parametrize("P", [16, 32, 512])
def test_reduce_of_partials_equals_decode(P):
    lens = [1, 15, 16, 17, 100, 600]
    r = _random_paged(10, len(lens), 4, 2, 64, "bf16", lens)
    args = (r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 4, 2, 64, "bf16", 0.125)
    ref = O.decode(*args)
    o, m, l, counts = O.partials(*args, partition_size=P)
    assert list(counts) == [-(-n // P) for n in lens]
    np.testing.assert_allclose(O.reduce(o, m, l, counts), ref, rtol=1e-12, atol=1e-14)


def test_partials_reject_bad_partition():
    r = _random_paged(10, 1, 2, 2, 64, "f32", [4])
    with pytest.raises(ValueError):
        O.partials(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 2, 2, 64, "f32", 0.125, 24)


# ---------------------------------------------------------------- cache write
def test_cache_write_is_a_bit_copy_and_touches_only_its_slots():
    rng = np.random.default_rng(13)
    H_kv, d, nblk = 2, 64, 4
    kp = _bf16(rng, nblk * H_kv * 16 * d)
    vp = _bf16(rng, nblk * H_kv * 16 * d)
    key = _bf16(rng, (3, H_kv, d))
    val = _bf16(rng, (3, H_kv, d))
    key[0, 0, 0] = 0x8000                           # -0.0 survives
    key[1, 1, 3] = 0x7FC1                           # a NaN payload survives
    slots = np.array([5, -1, 63], dtype=np.int64)
    k2, v2 = O.reshape_and_cache(kp, vp, key, val, slots, H_kv, d, "bf16", nblk)
    changed = np.flatnonzero(k2 != kp)
    assert changed.size <= 2 * H_kv * d
    for i, s in ((0, 5), (2, 63)):
        blk, off = divmod(s, 16)
        for h in range(H_kv):
            xs = np.arange(d)
            np.testing.assert_array_equal(k2[O.k_offset(blk, h, off, xs, H_kv, d, "bf16")], key[i, h])
            np.testing.assert_array_equal(v2[O.v_offset(blk, h, off, xs, H_kv, d, "bf16")], val[i, h])
    assert k2[O.k_offset(0, 0, 5, 0, H_kv, d, "bf16")] == 0x8000
    mask = np.ones(k2.size, bool)
    for s in (5, 63):
        blk, off = divmod(s, 16)
        for h in range(H_kv):
            mask[O.k_offset(blk, h, off, np.arange(d), H_kv, d, "bf16")] = False
    np.testing.assert_array_equal(k2[mask], kp[mask])


def test_cache_write_rejects_duplicates_and_out_of_range():
    kp = np.zeros(2 * 16 * 64, np.uint32)
    key = np.zeros((2, 1, 64), np.uint32)
    with pytest.raises(ValueError):
        O.reshape_and_cache(kp, kp, key, key, np.array([3, 3]), 1, 64, "f32", 2)
    with pytest.raises(ValueError):
        O.reshape_and_cache(kp, kp, key, key, np.array([3, 32]), 1, 64, "f32", 2)


def test_bytes_written_by_a_fresh_fill_equal_the_kv_formula():
    """A fresh fill of S tokens for B sequences writes 2*L*H_kv*d*b*S*B bytes (L=1)."""
    S, B, H_kv, d = 37, 3, 2, 64
    rng = np.random.default_rng(14)
    seq_k = [_bf16(rng, (S, H_kv, d)) for _ in range(B)]
    seq_v = [_bf16(rng, (S, H_kv, d)) for _ in range(B)]
    nb = O.blocks_needed(S)
    tables = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    kp, vp = _prefill_pool(seq_k, seq_v, tables, H_kv, d, "bf16", B * nb + 2)
    written = int(np.count_nonzero(kp != 0x7FC0) + np.count_nonzero(vp != 0x7FC0)) * 2
    assert written == O.kv_bytes(1, H_kv, d, 2, S, B)


# ---------------------------------------------------------------- sensitivity
def test_planted_mistakes_are_caught(monkeypatch):
    """Mistakes planted in the oracle (on the CPU) break at least one pin."""
    r = _random_paged(15, 2, 4, 2, 64, "bf16", [17, 40])
    scale = 0.125
    ref = _sdpa_reference(r["seq_k"], r["seq_v"], r["q"], 4, 2, 64, "bf16", scale)

    def run():
        return O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 4, 2, 64, "bf16", scale)

    np.testing.assert_allclose(run(), ref, rtol=1e-12, atol=1e-13)
    real_gather = O.pagedkv_oracle.gather_sequence

    # (1) drop the newest token (context length read as exclusive)
    def short(kp, vp, row, ctx, kvh, H_kv, d, dt, *scales):
        return real_gather(kp, vp, row, ctx - 1, kvh, H_kv, d, dt, *scales)
    monkeypatch.setattr(O.pagedkv_oracle, "gather_sequence", short)
    assert not np.allclose(run(), ref, rtol=1e-6)
    # (2) wrong KV head for a query head (h % H_kv instead of h // g)
    monkeypatch.setattr(O.pagedkv_oracle, "gather_sequence",
                        lambda kp, vp, row, ctx, kvh, H_kv, d, dt, *scales:
                        real_gather(kp, vp, row, ctx, (kvh + 1) % H_kv, H_kv, d, dt, *scales))
    assert not np.allclose(run(), ref, rtol=1e-6)
    monkeypatch.setattr(O.pagedkv_oracle, "gather_sequence", real_gather)
    # (3) transposed K/V layout
    real_k = O.pagedkv_oracle.k_offset
    monkeypatch.setattr(O.pagedkv_oracle, "k_offset",
                        lambda p, h, t, x, H_kv, d, dt: O.pagedkv_oracle.v_offset(p, h, t, x, H_kv, d, dt))
    kp_wrong = r["kp"]                                # written with the true layout
    got = O.decode(kp_wrong, r["vp"], r["q"], r["tables"], r["ctx"], 4, 2, 64, "bf16", scale)
    assert not np.allclose(got, ref, rtol=1e-6)
    monkeypatch.setattr(O.pagedkv_oracle, "k_offset", real_k)
    # (4) a scale of 1/d instead of 1/sqrt(d)
    got = O.decode(r["kp"], r["vp"], r["q"], r["tables"], r["ctx"], 4, 2, 64, "bf16", 1 / 64)
    assert not np.allclose(got, ref, rtol=1e-6)

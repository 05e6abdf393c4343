"""GPU parity of the block-management path: kv_copy_blocks, and a serving
scenario in which the native block manager (kv_bm_*) drives prompt admission
with prefix-cache hits, forks, copy-on-write appends and decode steps.

Each token's K/V rows are a fixed function of the token ids up to it, as in a
model, so a block reused through the prefix cache holds exactly the rows the
new sequence would have written.  At every round: the native manager agrees
with the oracle's model on every slot and copy; the GPU pools equal the
oracle's pools bit for bit; every live sequence's rows, gathered through its
table, are exactly its own token history; and decode over the batch matches
the float64 oracle within the bf16 tolerances.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from oracle.block_manager import BlockManagerModel
from workloads import configs as W

from _harness import assert_close, from_dev, log, to_dev

pytestmark = pytest.mark.gpu

BLOCK = 16


@pytest.mark.parametrize("dtype,H_kv,d", [("bf16", 2, 128), ("f32", 3, 64), ("fp8", 4, 128)])
def test_copy_blocks_is_a_bit_exact_block_copy(dtype, H_kv, d):
    rng = np.random.default_rng(3)
    num_blocks = 12
    n = num_blocks * H_kv * BLOCK * d
    bdt = W.bits_dtype(dtype)
    kp = rng.integers(0, np.iinfo(bdt).max, size=n, dtype=bdt, endpoint=True)
    vp = rng.integers(0, np.iinfo(bdt).max, size=n, dtype=bdt, endpoint=True)
    pool = P.KVPool(to_dev(kp), to_dev(vp), num_blocks, H_kv, d, dtype)
    src = np.array([3, 0, 7, -1, 5, 99, 4], dtype=np.int32)
    dst = np.array([9, 11, 1, 2, 5, 6, 10], dtype=np.int32)
    log(f"[gpu] copy_blocks {dtype} H_kv={H_kv} d={d}")
    P.kv_copy_blocks(pool, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    tile = H_kv * BLOCK * d
    ek, ev = kp.copy(), vp.copy()
    for s, t in zip(src, dst):
        if 0 <= s < num_blocks and 0 <= t < num_blocks and s != t:
            ek[t * tile:(t + 1) * tile] = kp[s * tile:(s + 1) * tile]
            ev[t * tile:(t + 1) * tile] = vp[s * tile:(s + 1) * tile]
    assert np.array_equal(from_dev(pool.k_cache, dtype), ek)
    assert np.array_equal(from_dev(pool.v_cache, dtype), ev)


class _Rows:
    """K/V rows of the token at the end of a token prefix (bf16 bits [H_kv, d])."""

    def __init__(self, H_kv, d):
        self.H_kv, self.d, self.memo = H_kv, d, {}

    def __call__(self, prefix):
        key = tuple(int(t) for t in prefix)
        if key not in self.memo:
            rng = np.random.default_rng([len(key)] + list(key[-24:]) + [hash(key) & 0xFFFFFFFF])
            x = rng.standard_normal((2, self.H_kv, self.d)).astype(np.float32)
            self.memo[key] = W.f32_to_bf16_bits(x)
        return self.memo[key]


def test_serving_scenario_with_prefix_hits_forks_and_copy_on_write():
    H, H_kv, d, num_blocks = 8, 2, 128, 48
    scale = 1 / np.sqrt(d)
    rows = _Rows(H_kv, d)
    n = num_blocks * H_kv * BLOCK * d
    nan = np.uint16(0x7FC0)
    kp = np.full(n, nan, np.uint16)
    vp = kp.copy()
    pool = P.KVPool(to_dev(kp), to_dev(vp), num_blocks, H_kv, d, "bf16")
    bm = P.BlockManager(num_blocks)
    model = BlockManagerModel(num_blocks)
    history = {}
    rng = np.random.default_rng(11)

    def write(seq, positions, slots):
        """Write the rows of seq's tokens at `positions` into `slots` (GPU and oracle)."""
        nonlocal kp, vp
        if not positions:
            return
        kv = np.stack([rows(history[seq][:p + 1]) for p in positions])   # [N, 2, H_kv, d]
        key, val = kv[:, 0].copy(), kv[:, 1].copy()
        sl = np.asarray(slots, dtype=np.int64)
        P.reshape_and_cache(pool, to_dev(key), to_dev(val), torch.from_numpy(sl).cuda())
        kp, vp = O.reshape_and_cache(kp, vp, key, val, sl, H_kv, d, "bf16", num_blocks)

    def admit(seq, prompt, salt=""):
        hits = bm.admit(seq, prompt, salt)
        assert hits == model.admit(seq, prompt, salt)
        history[seq] = list(prompt)
        table = bm.table(seq)
        assert table == model.table(seq)
        pos = list(range(hits, len(prompt)))
        write(seq, pos, [table[p // BLOCK] * BLOCK + p % BLOCK for p in pos])
        return hits

    def append(seq, token):
        nonlocal kp, vp
        slot, copy = bm.append(seq, token)
        assert (slot, copy) == model.append(seq, token)
        if copy is not None:
            P.kv_copy_blocks(pool, torch.tensor([copy[0]], dtype=torch.int32, device="cuda"),
                             torch.tensor([copy[1]], dtype=torch.int32, device="cuda"))
            tile = H_kv * BLOCK * d
            s, t = copy
            kp[t * tile:(t + 1) * tile] = kp[s * tile:(s + 1) * tile]
            vp[t * tile:(t + 1) * tile] = vp[s * tile:(s + 1) * tile]
        history[seq].append(token)
        write(seq, [len(history[seq]) - 1], [slot])
        return copy

    def check_round(label):
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(pool.k_cache, "bf16"), kp), f"{label}: K pool"
        assert np.array_equal(from_dev(pool.v_cache, "bf16"), vp), f"{label}: V pool"
        seqs = sorted(history)
        max_nb = max(len(bm.table(s)) for s in seqs)
        tables, lens = bm.batch_tables(seqs, max_nb)
        for b, s in enumerate(seqs):
            assert lens[b] == len(history[s])
            for kvh in range(H_kv):              # the table reaches exactly s's own rows
                K, V = O.gather_sequence(kp, vp, tables[b], int(lens[b]), kvh, H_kv, d, "bf16")
                want = np.stack([rows(history[s][:p + 1]) for p in range(len(history[s]))])
                np.testing.assert_array_equal(K, O.bits_to_f64(want[:, 0, kvh], "bf16"))
                np.testing.assert_array_equal(V, O.bits_to_f64(want[:, 1, kvh], "bf16"))
        q = W.f32_to_bf16_bits(rng.standard_normal((len(seqs), H, d)).astype(np.float32))
        out = torch.empty(len(seqs), H, d, dtype=torch.bfloat16, device="cuda").view(torch.int16)
        P.paged_attention_decode(pool, out, to_dev(q), torch.from_numpy(tables).cuda(),
                                 torch.from_numpy(lens).cuda(), int(lens.max()), scale)
        torch.cuda.synchronize()
        ref = {b: O.decode_sequence(kp, vp, q[b], tables[b], int(lens[b]), H, H_kv, d, "bf16", scale)
               for b in range(len(seqs))}
        err, rel = assert_close(from_dev(out, "bf16"), ref, "bf16", label)
        log(f"[gpu] {label}: {len(seqs)} sequences, free {bm.num_free()}, max-abs {err:.1e}")

    system = list(range(1000, 1040))
    log("[gpu] block-manager scenario")
    assert admit(1, system + [1, 2, 3]) == 0
    assert admit(2, system + [7, 8]) == 32
    bm.fork(2, 3); model.fork(2, 3); history[3] = list(history[2])
    bm.fork(1, 4); model.fork(1, 4); history[4] = list(history[1])
    check_round("after admits and forks")
    copies = 0
    for r in range(24):                          # crosses block boundaries, copies on write
        for s in (3, 2, 4, 1):
            copies += append(s, int(rng.integers(0, 50))) is not None
        if r % 8 == 7:
            check_round(f"round {r}")
    assert copies >= 2
    for s in (1, 4):
        bm.release(s); model.release(s); history.pop(s)
    assert admit(5, system + [9]) == 32          # the released prefix is still cached
    assert admit(6, [999] + system[1:]) == 0
    for r in range(10):
        for s in (2, 3, 5, 6):
            append(s, int(rng.integers(0, 50)))
    check_round("after release and re-admission")
    assert bm.num_free() == model.num_free()

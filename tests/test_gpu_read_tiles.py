"""GPU check of kv_read_tiles, the read-only pass the bench times as the
decode's bandwidth ceiling: it must read exactly the listed tiles of both
caches (entries outside the pool skipped), which the XOR checksum it returns
shows against the same XOR taken on the host over the same bytes.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_33_amd as P

from _harness import log, to_dev

pytestmark = pytest.mark.gpu


def _xor_words(buf: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(buf.view(np.uint32))) if buf.size else 0


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp8", 64), ("fp8", 128),
                                     ("f32", 128), ("int8", 128)])
@pytest.mark.parametrize("n,groups", [(0, 3), (1, 1), (37, 5), (5000, 512)])
def test_checksum_covers_exactly_the_listed_tiles(dtype, d, n, groups):
    H_kv, num_blocks = 4, 300
    elem = {"bf16": 2, "fp8": 1, "int8": 1, "f32": 4}[dtype]
    tile = 16 * d * elem
    nbytes = P.kv_pool_bytes(num_blocks, H_kv, d, dtype)
    rng = np.random.default_rng(n + groups + d)
    kp = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    vp = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    pool = P.KVPool(to_dev(kp), to_dev(vp), num_blocks, H_kv, d, dtype)
    tiles = rng.integers(-3, num_blocks * H_kv + 3, size=n).astype(np.int32)  # some outside
    sink = torch.full((groups,), -1, dtype=torch.int32, device="cuda")
    log(f"[gpu] read_tiles {dtype} d={d} n={n} groups={groups}")
    P.kv_read_tiles(pool, torch.from_numpy(tiles).cuda(), sink)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    want = 0
    for t in tiles:
        if 0 <= t < num_blocks * H_kv:
            want ^= _xor_words(kp[t * tile:(t + 1) * tile]) ^ _xor_words(vp[t * tile:(t + 1) * tile])
    assert got == want
    if n == 0:
        assert np.all(sink.cpu().numpy() == 0)   # every work-group stores its (empty) XOR

"""GPU parity at the batch sizes where the launch's bookkeeping changes form.

Single pass: work-groups take sequences longest first, an order every
work-group derives from the lengths for batches of up to 4,096 sequences, and
index order above that.  Split mode: the work list of partitions holds up to
4,096 sequences (the API refuses more; tests/test_abi.py).  Each case runs a
batch at or just past its limit, with short random lengths (1 to 40 tokens,
so many sequences share a length bucket) and small heads, through the
vector-ALU kernel (MHA) and the matrix-core kernel (GQA), and compares the
whole step with the oracle: slots and pools bit for bit, every output within
the bf16 tolerance.
"""
import numpy as np
import pytest

from workloads import configs as W

from _harness import single_step_case

pytestmark = pytest.mark.gpu


def _workload(B: int, H: int, H_kv: int, seed: int) -> W.Workload:
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 41, size=B).tolist()
    return W.scattered_workload(f"batch{B}", "bf16", B=B, H=H, H_kv=H_kv, d=64,
                                context_lens=lens, seed=seed)


@pytest.mark.parametrize("B", [4096, 4100])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2)])
def test_single_pass_at_the_ordering_limit(B, H, H_kv):
    """4,096 sequences: the longest-first order over the whole batch; 4,100:
    index order.  Either way each sequence is computed exactly once."""
    w = _workload(B, H, H_kv, seed=B + 7 * H)
    single_step_case(w, 0, label=f"single pass B={B} H={H}/{H_kv}")


@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2)])
def test_split_at_the_work_list_limit(H, H_kv):
    """4,096 sequences in 16-token partitions: the work list's prefix sums fill
    their LDS array, and sequences of one partition write their output
    directly while the others go through the reduce."""
    w = _workload(4096, H, H_kv, seed=31 + H)
    single_step_case(w, 16, label=f"split B=4096 H={H}/{H_kv}")

"""Pins of the oracle's element decoding (CPU).

Every attention pin widens stored bit patterns through `bits_to_f64`, so that
function is pinned here against decoders that share nothing with it: torch's
own bfloat16, float32 and int8 dtypes, reinterpreting the same bits.  A
decoder that read bf16 bits as float16, or shifted them by the wrong amount,
fails these pins (planted below).
"""
import numpy as np
import pytest
import torch

import oracle as O


def _torch_widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Independent decoder: reinterpret the bits as a torch dtype, widen to float64."""
    view = {"bf16": (np.int16, torch.bfloat16), "f32": (np.int32, torch.float32),
            "int8": (np.int8, torch.int8)}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(bits).view(view[0]).copy())
    return t.view(view[1]).to(torch.float64).numpy()


def _same_values(a: np.ndarray, b: np.ndarray) -> bool:
    """Equal value for value, NaN matching NaN, and the sign of zero kept."""
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    if not np.array_equal(nan_a, nan_b):
        return False
    fa, fb = a[~nan_a], b[~nan_b]
    return bool(np.array_equal(fa, fb) and np.array_equal(np.signbit(fa), np.signbit(fb)))


def _all_bf16_patterns() -> np.ndarray:
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _bf16_pin_holds(decode) -> bool:
    bits = _all_bf16_patterns()
    return _same_values(decode(bits, "bf16"), _torch_widen(bits, "bf16"))


def test_bf16_widening_matches_torch_for_every_pattern():
    assert _bf16_pin_holds(O.bits_to_f64)


def test_bf16_widening_spot_values():
    # values the format fixes: 1.0 = 0x3F80, -2.0 = 0xC000, the smallest
    # subnormal 2^-133 = 0x0001, the largest finite (2 - 2^-7)*2^127 = 0x7F7F
    got = O.bits_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x7F80, 0xFF80], np.uint16), "bf16")
    assert got[0] == 1.0 and got[1] == -2.0
    assert got[2] == 2.0 ** -133
    assert got[3] == (2 - 2 ** -7) * 2.0 ** 127
    assert got[4] == np.inf and got[5] == -np.inf


def test_f32_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = np.concatenate([
        rng.integers(0, 1 << 32, size=1 << 18, dtype=np.uint64).astype(np.uint32),
        np.array([0, 0x80000000, 1, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000],
                 np.uint32)])
    assert _same_values(O.bits_to_f64(bits, "f32"), _torch_widen(bits, "f32"))


def test_int8_widening_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = O.bits_to_f64(codes, "int8")
    assert _same_values(got, _torch_widen(codes, "int8"))
    assert got[0x7F] == 127 and got[0x80] == -128 and got[0xFF] == -1


def test_fp8_widening_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same_values(O.bits_to_f64(codes, "fp8"), want)


@pytest.mark.parametrize("mistake", ["float16", "shift15", "low-half"])
def test_planted_bf16_mistakes_fail_the_pin(mistake):
    def planted(bits, dtype):
        b = np.asarray(bits)
        with np.errstate(invalid="ignore"):
            if mistake == "float16":          # bf16 bits read as IEEE half
                return b.astype(np.uint16).view(np.float16).astype(np.float64)
            if mistake == "shift15":          # widened by a wrong shift
                return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
            # the 16 bits placed in the low half of the float32
            return b.astype(np.uint32).view(np.float32).astype(np.float64)
    assert not _bf16_pin_holds(planted)

"""Pins for the oracle's 16-bit conversions.

The oracle writes its binary16 and bfloat16 round-to-nearest-even conversions
from the IEEE-754 definitions; here they are checked over every binary32 bit
pattern against library routines that implement the same standard: numpy's
float32 -> float16 cast and torch's float32 -> bfloat16 cast (both round to
nearest even).  The payload parameters are half precision ([JP] section
'よくある質問'); the message is 16-bit (bf16) in and out.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O

CHUNK = 1 << 25


def _nan16(h, exp_mask, man_mask):
    return ((h & exp_mask) == exp_mask) & ((h & man_mask) != 0)


def _sweep(ours_fn, torch_dtype, exp_mask, man_mask):
    """Compare a conversion with torch's over all 2^32 binary32 patterns.
    NaN inputs only need to give NaN outputs (payloads are not compared)."""
    base = np.arange(CHUNK, dtype=np.uint32)

    def one(start):
        u = base + np.uint32(start)
        f = u.view(np.float32)
        ours = ours_fn(f)
        ref = torch.from_numpy(f).to(torch_dtype).view(torch.int16).numpy().view(np.uint16)
        bad = np.nonzero(ours != ref)[0]
        if bad.size:
            both_nan = _nan16(ours[bad], exp_mask, man_mask) & _nan16(ref[bad], exp_mask, man_mask)
            bad = bad[~both_nan]
        return None if bad.size == 0 else int(u[bad[0]])

    with ThreadPoolExecutor(max_workers=4) as ex:
        for first_bad in ex.map(one, range(0, 1 << 32, CHUNK)):
            assert first_bad is None, f"first mismatch at f32 bits {first_bad:#010x}"


def test_f32_to_f16_exhaustive():
    _sweep(O.f32_to_f16_bits, torch.float16, 0x7C00, 0x03FF)


def test_f16_to_f32_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_exhaustive():
    _sweep(O.f32_to_bf16_bits, torch.bfloat16, 0x7F80, 0x007F)


@pytest.mark.parametrize("val,bits", [
    (65504.0, 0x7BFF),            # largest finite half
    (65519.99, 0x7BFF),           # rounds down, still finite
    (65520.0, 0x7C00),            # halfway to the next binade: ties to even -> infinity
    (2.0 ** -24, 0x0001),         # smallest subnormal half
    (2.0 ** -25, 0x0000),         # exact tie between 0 and 2^-24 -> even (0)
    (3 * 2.0 ** -26, 0x0001),     # above the tie
    (2.0 ** -14, 0x0400),         # smallest normal half
    (-0.0, 0x8000),
    (1.0 + 2.0 ** -11, 0x3C00),   # tie -> even significand
    (1.0 + 3 * 2.0 ** -11, 0x3C02),
])
def test_f32_to_f16_special_values(val, bits):
    f = np.array([val], np.float32)
    assert int(O.f32_to_f16_bits(f)[0]) == bits
    with np.errstate(over="ignore"):
        assert int(f.astype(np.float16).view(np.uint16)[0]) == bits

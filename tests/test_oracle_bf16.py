"""Pins of the oracle's bfloat16 conversions (oracle/quant.py: bf16_bits,
as_f32 on uint16 bit patterns) against an independent implementation:
torch's own float32 <-> bfloat16 casts on the CPU.

The quantised-pool oracle writes bf16(code * scale) rows from bf16_bits and
reads bf16 queries and rows through as_f32, so every expected value of the
quantised gather and decode rests on these two.  The reading of the pages'
precision (outputs are rounded to nearest, ties to even, from float32) is
checked here against a library routine rather than against a retyped bit
formula:

  * as_f32 is compared with torch's bf16 -> float32 cast on all 65536 bit
    patterns (exhaustive, NaN payloads included, compared as bits);
  * bf16_bits is compared with torch's float32 -> bf16 cast on every exact
    tie (low half 0x8000) and its two neighbours (0x7FFF, 0x8001) above each
    finite bf16 value of either sign, on 2^20 random finite float32 bit
    patterns, subnormals, and values at the top of the bf16 range (where
    rounding up overflows to infinity);
  * three planted mistakes -- truncation, ties away from zero, and ties to
    odd -- each fail the pin.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import quant as Q


def torch_bf16_bits(x):
    """float32 -> bf16 bit patterns by torch's cast (the independent side)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def finite_bf16_patterns():
    """Every bf16 bit pattern whose value is finite (both signs)."""
    p = np.arange(1 << 16, dtype=np.uint32)
    return p[(p & 0x7F80) != 0x7F80]


def cases():
    """float32 inputs that cover each rounding situation."""
    hi = finite_bf16_patterns() << 16
    ties = [hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi | 0x0001, hi]
    rng = np.random.default_rng(20260)
    r = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    r = r[(r & 0x7F800000) != 0x7F800000]                      # finite only
    sub = rng.integers(1, 1 << 23, size=4096, dtype=np.uint32)  # float32 subnormals
    top = np.array([0x7F7F0000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF,
                    0x7F7E8000, 0x7F7F8001], np.uint32)
    u = np.concatenate(ties + [r, sub, sub | 0x80000000, top, top | 0x80000000])
    return u.view(np.float32)


def check_bf16_bits(fn):
    """Names of the case families where fn differs from torch's cast."""
    x = cases()
    want = torch_bf16_bits(x)
    got = np.asarray(fn(x)).astype(np.uint16)
    bad = []
    if not np.array_equal(got, want):
        u = x.view(np.uint32)
        low = u & 0xFFFF
        diff = got != want
        if np.any(diff & (low == 0x8000)):
            bad.append("exact ties")
        if np.any(diff & (low != 0x8000)):
            bad.append("non-ties")
    return bad


def test_as_f32_matches_torch_on_every_bf16_pattern():
    p = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    got = Q.as_f32(p)
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), want.numpy().view(np.uint32))


def test_bf16_bits_matches_torch():
    assert check_bf16_bits(Q.bf16_bits) == []


def test_bf16_bits_worked_ties():
    # 1 + 2^-8 sits halfway between bf16 1.0 (even) and 1 + 2^-7: down to even;
    # 1 + 3 * 2^-8 sits halfway between 1 + 2^-7 (odd) and 1 + 2^-6: up to even
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), -(1 + 3 * 2.0 ** -8)],
                 np.float32)
    assert list(Q.bf16_bits(x)) == [0x3F80, 0x3F82, 0xBF80, 0xBF82]
    assert list(torch_bf16_bits(x)) == [0x3F80, 0x3F82, 0xBF80, 0xBF82]


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)


def mutant_truncate(x):
    return (_bits(x) >> 16).astype(np.uint16)


def mutant_ties_away(x):
    return ((_bits(x) + 0x8000) >> 16).astype(np.uint16)


def mutant_ties_odd(x):
    u = _bits(x)
    return ((u + 0x7FFF + (((u >> 16) & 1) ^ 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("mutant", [mutant_truncate, mutant_ties_away, mutant_ties_odd])
def test_planted_bf16_mistakes_fail(mutant):
    assert check_bf16_bits(mutant) != []

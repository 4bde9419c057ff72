"""Pins for the oracle's fp16 conversions against numpy's binary16 type and a
brute-force search over every finite fp16 value."""

import numpy as np
import pytest


def _all_finite_f16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    keep = np.isfinite(vals)
    return bits[keep], vals[keep]


def test_decode_every_bit_pattern(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle_mod.f16_to_f64(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # signed zeros decode with their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _rn_cases():
    rng = np.random.default_rng(7)
    cases = []
    # random fp32 bit patterns over the fp16-relevant exponent range
    e = rng.integers(127 - 30, 127 + 17, size=400000).astype(np.uint32)
    m = rng.integers(0, 1 << 23, size=400000).astype(np.uint32)
    s = rng.integers(0, 2, size=400000).astype(np.uint32)
    cases.append(((s << 31) | (e << 23) | m).view(np.float32))
    # exact midpoints between neighbouring fp16 values (ties) and their fp32 neighbours
    _, vals = _all_finite_f16()
    v = np.unique(vals)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    cases += [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))]
    cases.append(np.array([0.0, -0.0, 65504.0, 65519.0, 65519.996, 65520.0, -65520.0, 1e9, -1e9,
                           2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25],
                          dtype=np.float32))
    return np.concatenate(cases)


def test_round_nearest_even_matches_numpy(oracle_mod):
    x = _rn_cases()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle_mod.f16_rn(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("mode", ["rd", "ru"])
def test_directed_rounding_brute_force(oracle_mod, mode):
    """RD(x) = largest finite fp16 <= x, RU(x) = smallest finite fp16 >= x,
    found by binary search in the sorted table of every finite fp16."""
    _, vals = _all_finite_f16()
    table = np.unique(vals)
    x = _rn_cases()
    x = x[np.abs(x.astype(np.float64)) <= 65504.0]
    x64 = x.astype(np.float64)
    if mode == "rd":
        ref = table[np.searchsorted(table, x64, side="right") - 1]
        got = oracle_mod.f16_to_f64(oracle_mod.f16_rd(x))
    else:
        ref = table[np.searchsorted(table, x64, side="left")]
        got = oracle_mod.f16_to_f64(oracle_mod.f16_ru(x))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_directed_rounding_zero_signs(oracle_mod):
    tiny = np.array([1e-9, -1e-9, 0.0, -0.0], dtype=np.float32)
    rd = oracle_mod.f16_rd(tiny)
    ru = oracle_mod.f16_ru(tiny)
    assert list(rd) == [0x0000, 0x8001, 0x0000, 0x8000]
    assert list(ru) == [0x0001, 0x8000, 0x0000, 0x8000]

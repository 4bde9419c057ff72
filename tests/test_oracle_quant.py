"""Pins for the oracle's group-affine int4 quantiser and nibble packing.

Each check rests on something other than the quantiser's own formula: words
built by hand, groups that lie exactly on a grid, the half-step error bound,
a brute-force nearest-level search, and degenerate groups."""

import numpy as np
import pytest

import kvq_synth


def test_pack_hand_built_words(oracle_mod):
    # codes 0..7 in dimension order read back as hex digits, lowest first
    assert oracle_mod.pack_row(np.arange(8)).tolist() == [0x76543210]
    assert oracle_mod.pack_row(np.arange(8)[::-1]).tolist() == [0x01234567]
    # every code at every position
    for pos in range(8):
        for code in range(16):
            c = np.zeros(8, dtype=np.uint8)
            c[pos] = code
            assert oracle_mod.pack_row(c).tolist() == [code << (4 * pos)]
    # second word holds dimensions 8..15
    c = np.zeros(16, dtype=np.uint8)
    c[9] = 0xA
    assert oracle_mod.pack_row(c).tolist() == [0, 0xA0]


def test_unpack_roundtrip(oracle_mod):
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, size=256).astype(np.uint8)
    assert np.array_equal(oracle_mod.unpack_row(oracle_mod.pack_row(c)), c)
    w = rng.integers(0, 2 ** 32, size=32, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle_mod.pack_row(oracle_mod.unpack_row(w)), w)


@pytest.mark.parametrize("seed", range(20))
def test_lossless_on_grid(oracle_mod, seed):
    """A group whose values are exactly b + k*s (b, s fp16, codes 0 and 15
    both present) is recovered exactly: codes k, scale s, bias b."""
    rng = np.random.default_rng(seed)
    G = 64
    s = np.float16(rng.integers(1, 2048) * 2.0 ** rng.integers(-12, -4))
    b = np.float16(rng.integers(-2048, 2048) * 2.0 ** rng.integers(-8, -1))
    k = rng.integers(0, 16, size=G)
    k[rng.integers(0, G)] = 0
    k[rng.integers(0, G)] = 15
    if not (k == 0).any() or not (k == 15).any():
        k[0], k[1] = 0, 15
    x = float(b) + k * float(s)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)  # exact in fp32
    codes, sbits, bbits = oracle_mod.quantize_group(x.astype(np.float32))
    assert sbits == int(np.float16(s).view(np.uint16))
    assert bbits == int(np.float16(b).view(np.uint16)) or (float(b) == 0 and bbits == 0)
    assert np.array_equal(codes, k)


def _groups():
    """Groups of 64 with the workloads' distributions plus hard cases."""
    out = []
    out.append(kvq_synth.normal((4000, 64), [99, 0]))                                   # fp32 N(0,1)
    out.append(kvq_synth.normal((4000, 64), [99, 1]).astype(np.float16).astype(np.float32))
    out.append(kvq_synth.student_t((4000, 64), 3.0, [99, 2]) * np.float32(20))           # outliers
    out.append(np.float32(100) + np.float32(1e-3) * kvq_synth.normal((2000, 64), [99, 3]))  # narrow, offset
    out.append(np.float32(1e-6) * kvq_synth.normal((2000, 64), [99, 4]))                # near fp16 underflow
    out.append(np.float32(3e4) * kvq_synth.uniform((2000, 64), -1, 1, [99, 5]))         # near fp16 max
    return np.concatenate(out).astype(np.float32)


def test_error_bound_and_range(oracle_mod):
    """bias <= min, max <= bias + 15*scale, and |x - x^| <= scale/2 up to
    the fp32 rounding of (x - bias)/scale."""
    x = _groups()
    words, sc, bi = oracle_mod.quantize_rows(x, 64)
    s = oracle_mod.f16_to_f64(sc)[:, 0]
    b = oracle_mod.f16_to_f64(bi)[:, 0]
    x64 = x.astype(np.float64)
    assert np.all(b <= x64.min(axis=1))
    assert np.all(x64.max(axis=1) <= b + 15 * s * (1 + 2.0 ** -20))
    xh = oracle_mod.dequantize_rows(words, sc, bi, 64)
    err = np.abs(xh - x64).max(axis=1)
    assert np.all(err <= s / 2 * (1 + 2.0 ** -17) + 1e-300)
    assert np.all(s > 0)


def test_nearest_level_brute_force(oracle_mod):
    """Each code is a nearest level among all 16 (ties within fp32 rounding
    may go either way)."""
    x = _groups()[::7]
    words, sc, bi = oracle_mod.quantize_rows(x, 64)
    s = oracle_mod.f16_to_f64(sc)[:, 0:1]
    b = oracle_mod.f16_to_f64(bi)[:, 0:1]
    codes = np.stack([oracle_mod.unpack_row(w) for w in words]).astype(np.float64)
    levels = b[:, :, None] + np.arange(16)[None, None, :] * s[:, :, None]  # [rows,1,16]
    dist = np.abs(x.astype(np.float64)[:, :, None] - levels)
    best = dist.min(axis=2)
    chosen = np.abs(x.astype(np.float64) - (b + codes * s))
    assert np.all(chosen <= best + s * 2.0 ** -17)


def test_degenerate_groups(oracle_mod):
    # all equal and fp16-exact: zero scale, bias = value, codes 0, exact
    for v in (0.0, 1.5, -3.25, 65504.0, -65504.0, 2.0 ** -24):
        codes, sbits, bbits = oracle_mod.quantize_group(np.full(64, v, dtype=np.float32))
        assert sbits == 0 and not codes.any()
        assert oracle_mod.f16_to_f64(np.array([bbits], dtype=np.uint16))[0] == v
    # all -0.0: bias stored as +0
    codes, sbits, bbits = oracle_mod.quantize_group(np.full(64, -0.0, dtype=np.float32))
    assert (sbits, bbits) == (0, 0)
    # all equal but not fp16-exact: bias below, small positive scale, within bound
    x = np.full(64, 0.1, dtype=np.float32)
    codes, sbits, bbits = oracle_mod.quantize_group(x)
    b = oracle_mod.f16_to_f64(np.array([bbits], dtype=np.uint16))[0]
    s = oracle_mod.f16_to_f64(np.array([sbits], dtype=np.uint16))[0]
    assert b < 0.1 and s > 0
    assert abs(codes[0] * s + b - float(np.float32(0.1))) <= s / 2 * (1 + 2.0 ** -17)


def test_fp16_inputs_keep_exact_min(oracle_mod):
    """For fp16 inputs the bias is the group minimum itself."""
    x = kvq_synth.normal((500, 64), [98, 0]).astype(np.float16)
    _, _, bi = oracle_mod.quantize_rows(x, 64)
    mn = x.astype(np.float64).min(axis=1)
    got = oracle_mod.f16_to_f64(bi)[:, 0]
    assert np.array_equal(got, mn + 0.0)  # -0.0 min is stored as +0


def test_rows_layout_groups(oracle_mod):
    """quantize_rows packs groups in dimension order: group g of row r is
    quantize_group on x[r, g*G:(g+1)*G]."""
    x = kvq_synth.normal((3, 256), [97, 0])
    words, sc, bi = oracle_mod.quantize_rows(x, 64)
    for r in range(3):
        codes = oracle_mod.unpack_row(words[r])
        for g in range(4):
            c, s, b = oracle_mod.quantize_group(x[r, g * 64:(g + 1) * 64])
            assert np.array_equal(codes[g * 64:(g + 1) * 64], c)
            assert (sc[r, g], bi[r, g]) == (s, b)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bias,step", [(0.0, 1.0), (-4.0, 0.5), (3.0, 0.25)])
def test_exact_ties_round_to_even(oracle_mod, bits, bias, step):
    """Reading R3 of the code rounding (the pages name no rule): a quotient
    (x - bias) / scale that lies exactly halfway between two codes takes the
    even one. The group holds its own minimum (bias, fp16-exact, so the bias
    is that value) and maximum bias + levels * step (scale exactly step, a
    power of two, so every quotient below is exact in fp32), and every
    half-integer quotient k + 1/2 in between. Rounding half away from zero
    would give k + 1 for every even k and fails here."""
    levels = (1 << bits) - 1
    half = np.arange(levels, dtype=np.float64) + 0.5  # 0.5, 1.5, ..., levels - 0.5
    G = 64 if bits == 4 else 256
    members = np.concatenate([[0.0, float(levels)], half])
    members = np.resize(members, G)  # both ends first, ties fill the rest
    x = bias + members * step
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    codes, sbits, bbits = oracle_mod.quantize_group(x.astype(np.float32), bits)
    s = oracle_mod.f16_to_f64(np.array([sbits], dtype=np.uint16))[0]
    b = oracle_mod.f16_to_f64(np.array([bbits], dtype=np.uint16))[0]
    assert (s, b) == (step, bias)
    # k + 1/2 -> k when k is even, k + 1 when k is odd
    k = np.floor(members)
    expect = np.where(members == k, k, np.where(k % 2 == 0, k, k + 1))
    assert np.array_equal(codes.astype(np.float64), expect)
    # spot values named in the rule: 0.5 -> 0, 2.5 -> 2, 14.5 -> 14 (and 1.5 -> 2)
    by_member = {float(m): int(c) for m, c in zip(members, codes)}
    assert by_member[0.5] == 0 and by_member[1.5] == 2 and by_member[2.5] == 2 and by_member[14.5] == 14

"""Pins for the oracle's 8-bit variant of the group-affine quantiser (the
Gemma page's "What I Tried" table lists an int8 KV cache; the blog's decode
driver takes 4 or 8 KV bits): the same rule with 255 steps, codes 0..255
packed four to a word, lowest byte first.

Each check rests on something other than the quantiser's own formula: words
built by hand, groups that lie exactly on the 256-level grid, the half-step
error bound, a brute-force nearest-level search over all 256 levels,
degenerate groups, the fixed ratio between the int4 and int8 steps, and
torch's float64 SDPA on the dequantised int8 cache."""

import numpy as np
import pytest
import torch

import kvq_synth
from test_oracle_quant import _groups


def test_pack_hand_built_words(oracle_mod):
    assert oracle_mod.pack_row(np.arange(4), bits=8).tolist() == [0x03020100]
    assert oracle_mod.pack_row(np.array([0xFF, 0x80, 0x01, 0x7F]), bits=8).tolist() == [0x7F0180FF]
    for pos in range(4):
        for code in (1, 0x5A, 0x80, 0xFF):
            c = np.zeros(4, dtype=np.uint8)
            c[pos] = code
            assert oracle_mod.pack_row(c, bits=8).tolist() == [code << (8 * pos)]
    c = np.zeros(8, dtype=np.uint8)
    c[5] = 0xC3  # second word holds dimensions 4..7
    assert oracle_mod.pack_row(c, bits=8).tolist() == [0, 0xC300]


def test_unpack_roundtrip(oracle_mod):
    rng = np.random.default_rng(4)
    c = rng.integers(0, 256, size=256).astype(np.uint8)
    w = oracle_mod.pack_row(c, bits=8)
    assert w.size == 64
    assert np.array_equal(oracle_mod.unpack_row(w, bits=8), c)
    w = rng.integers(0, 2 ** 32, size=32, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle_mod.pack_row(oracle_mod.unpack_row(w, bits=8), bits=8), w)
    # the same word read as nibbles and as bytes: byte j = nibbles 2j, 2j+1
    nib = oracle_mod.unpack_row(w, bits=4).astype(np.int64)
    byt = oracle_mod.unpack_row(w, bits=8).astype(np.int64)
    assert np.array_equal(byt, nib[0::2] + 16 * nib[1::2])


def test_bad_bits_rejected(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.quantize_group(np.zeros(64, dtype=np.float32), bits=2)
    with pytest.raises(ValueError):
        oracle_mod.Cache(1, 1, 64, 8, 64, bits=16)


@pytest.mark.parametrize("seed", range(20))
def test_lossless_on_grid(oracle_mod, seed):
    """Values exactly b + k*s (b, s fp16; codes 0 and 255 both present) come
    back as codes k, scale s, bias b."""
    rng = np.random.default_rng(100 + seed)
    G = 64
    s = np.float16(rng.integers(1, 2048) * 2.0 ** rng.integers(-12, -4))
    b = np.float16(rng.integers(-2048, 2048) * 2.0 ** rng.integers(-8, -1))
    k = rng.integers(0, 256, size=G)
    k[0], k[1] = 0, 255
    rng.shuffle(k)
    x = float(b) + k * float(s)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)  # exact in fp32
    codes, sbits, bbits = oracle_mod.quantize_group(x.astype(np.float32), bits=8)
    assert sbits == int(np.float16(s).view(np.uint16))
    assert bbits == int(np.float16(b).view(np.uint16)) or (float(b) == 0 and bbits == 0)
    assert np.array_equal(codes, k)


def test_error_bound_and_range(oracle_mod):
    """bias <= min, max <= bias + 255*scale, and |x - x^| <= scale/2 up to
    the fp32 rounding of (x - bias)/scale (at most about 2^-15 of a step for
    quotients below 256)."""
    x = _groups()
    words, sc, bi = oracle_mod.quantize_rows(x, 64, bits=8)
    assert words.shape == (x.shape[0], 16)
    s = oracle_mod.f16_to_f64(sc)[:, 0]
    b = oracle_mod.f16_to_f64(bi)[:, 0]
    x64 = x.astype(np.float64)
    assert np.all(b <= x64.min(axis=1))
    assert np.all(x64.max(axis=1) <= b + 255 * s * (1 + 2.0 ** -20))
    xh = oracle_mod.dequantize_rows(words, sc, bi, 64, bits=8)
    err = np.abs(xh - x64).max(axis=1)
    assert np.all(err <= s / 2 * (1 + 2.0 ** -13) + 1e-300)
    assert np.all(s > 0)


def test_nearest_level_brute_force(oracle_mod):
    """Each code is a nearest level among all 256 (near-ties within the fp32
    rounding may go either way)."""
    x = _groups()[::11]
    words, sc, bi = oracle_mod.quantize_rows(x, 64, bits=8)
    s = oracle_mod.f16_to_f64(sc)[:, 0:1]
    b = oracle_mod.f16_to_f64(bi)[:, 0:1]
    codes = np.stack([oracle_mod.unpack_row(w, bits=8) for w in words]).astype(np.float64)
    levels = b[:, :, None] + np.arange(256)[None, None, :] * s[:, :, None]
    best = np.abs(x.astype(np.float64)[:, :, None] - levels).min(axis=2)
    chosen = np.abs(x.astype(np.float64) - (b + codes * s))
    assert np.all(chosen <= best + s * 2.0 ** -14)


def test_step_ratio_to_int4(oracle_mod):
    """Both steps are the group range over the level count, rounded up to
    fp16, so where both are normal fp16 numbers the int4 step is 17 times
    the int8 one up to those roundings (255 / 15 = 17); a subnormal int8 step
    is the range over 255 rounded up to the 2^-24 quantum. The bias is the
    same."""
    x = _groups()[::5]
    _, s4, b4 = oracle_mod.quantize_rows(x, 64, bits=4)
    _, s8, b8 = oracle_mod.quantize_rows(x, 64, bits=8)
    assert np.array_equal(b4, b8)
    a = oracle_mod.f16_to_f64(s4)[:, 0]
    b = oracle_mod.f16_to_f64(s8)[:, 0]
    normal = b >= 2.0 ** -14
    assert normal.sum() > 3000 and (~normal).sum() > 100
    r = a[normal] / (17 * b[normal])
    assert np.all(np.abs(r - 1) <= 2.0 ** -9)
    rng8 = (x.astype(np.float64).max(axis=1) - oracle_mod.f16_to_f64(b8)[:, 0])[~normal] / 255
    assert np.all(b[~normal] >= rng8 * (1 - 2.0 ** -22))
    assert np.all(b[~normal] < rng8 + 2.0 ** -24)


def test_degenerate_groups(oracle_mod):
    for v in (0.0, 1.5, -3.25, 65504.0, -65504.0, 2.0 ** -24):
        codes, sbits, bbits = oracle_mod.quantize_group(np.full(64, v, dtype=np.float32), bits=8)
        assert sbits == 0 and not codes.any()
        assert oracle_mod.f16_to_f64(np.array([bbits], dtype=np.uint16))[0] == v
    codes, sbits, bbits = oracle_mod.quantize_group(np.full(64, -0.0, dtype=np.float32), bits=8)
    assert (sbits, bbits) == (0, 0)
    # two values: min -> code 0, max -> code 255 exactly when the step is exact
    x = np.zeros(64, dtype=np.float32)
    x[7] = 255.0
    codes, sbits, bbits = oracle_mod.quantize_group(x, bits=8)
    assert (sbits, bbits) == (int(np.float16(1.0).view(np.uint16)), 0)
    assert codes[7] == 255 and codes.sum() == 255


def test_rows_layout_groups(oracle_mod):
    x = kvq_synth.normal((3, 256), [96, 0])
    words, sc, bi = oracle_mod.quantize_rows(x, 64, bits=8)
    assert words.shape == (3, 64)
    for r in range(3):
        codes = oracle_mod.unpack_row(words[r], bits=8)
        for g in range(4):
            c, s, b = oracle_mod.quantize_group(x[r, g * 64:(g + 1) * 64], bits=8)
            assert np.array_equal(codes[g * 64:(g + 1) * 64], c)
            assert (sc[r, g], bi[r, g]) == (s, b)


def _deq(oracle_mod, c, S):
    kd = oracle_mod.dequantize_rows(c.k_q[:, :, :S], c.k_scale[:, :, :S], c.k_bias[:, :, :S], c.G, c.bits)
    vd = oracle_mod.dequantize_rows(c.v_q[:, :, :S], c.v_scale[:, :, :S], c.v_bias[:, :, :S], c.G, c.bits)
    return kd, vd


@pytest.mark.parametrize("hq,hkv,d,s,alpha,G", [(8, 2, 128, 1024, 1 / np.sqrt(128), 64),
                                                (4, 4, 64, 37, 0.3, 32), (8, 1, 256, 300, 1.0, 128)])
def test_attention_matches_torch_sdpa(oracle_mod, hq, hkv, d, s, alpha, G):
    q = kvq_synth.normal((1, hq, d), [54, hq, d, s, 0])
    k = kvq_synth.normal((1, hkv, s, d), [54, hq, d, s, 1])
    v = kvq_synth.normal((1, hkv, s, d), [54, hq, d, s, 2])
    c = oracle_mod.Cache(1, hkv, d, s + 3, G, bits=8)
    assert c.k_q.shape == (1, hkv, s + 3, d // 4)
    c.append(k, v, 0)
    kd, vd = _deq(oracle_mod, c, s)
    got = oracle_mod.sdpa(c, s, q, alpha)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, torch.from_numpy(kd), torch.from_numpy(vd),
                                                           scale=alpha, enable_gqa=hq != hkv)[:, :, 0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # int8 sits far closer to the unquantised attention than int4 does
    exact = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(k.astype(np.float64)), torch.from_numpy(v.astype(np.float64)), scale=alpha,
        enable_gqa=hq != hkv)[:, :, 0].numpy()
    c4 = oracle_mod.Cache(1, hkv, d, s, G)
    c4.append(k, v, 0)
    e8 = np.linalg.norm(got - exact)
    e4 = np.linalg.norm(oracle_mod.sdpa(c4, s, q, alpha) - exact)
    assert e8 < e4 / 8


def test_partials_combine_to_sdpa(oracle_mod):
    q = kvq_synth.normal((1, 8, 128), [55, 0])
    k = kvq_synth.normal((1, 2, 1300, 128), [55, 1]).astype(np.float16)
    v = kvq_synth.normal((1, 2, 1300, 128), [55, 2]).astype(np.float16)
    c = oracle_mod.Cache(1, 2, 128, 1300, 64, bits=8)
    c.append(k, v, 0)
    m, l, acc = oracle_mod.sdpa_partials(c, 1300, q, 0.09, 512)
    assert m.shape[-1] == 3
    np.testing.assert_allclose(oracle_mod.combine_partials(m, l, acc), oracle_mod.sdpa(c, 1300, q, 0.09),
                               rtol=1e-12, atol=1e-14)


def test_constant_v_gives_that_row(oracle_mod):
    k = kvq_synth.normal((1, 2, 600, 128), [56, 1])
    row = kvq_synth.normal((128,), [56, 2]).astype(np.float16)
    v = np.broadcast_to(row, (1, 2, 600, 128)).copy()
    q = kvq_synth.normal((1, 8, 128), [56, 0])
    c = oracle_mod.Cache(1, 2, 128, 600, 64, bits=8)
    c.append(k, v, 0)
    got = oracle_mod.sdpa(c, 600, q, 1.0)
    vrow = oracle_mod.dequantize_rows(c.v_q[0, 0, :1], c.v_scale[0, 0, :1], c.v_bias[0, 0, :1], 64, 8)[0]
    # every row is the same dequantised row, whatever the weights
    np.testing.assert_allclose(got, np.broadcast_to(vrow, got.shape), rtol=0, atol=1e-12)

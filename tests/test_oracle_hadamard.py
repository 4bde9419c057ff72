"""Pins for the oracle's Hadamard rotation (the rotated-cache variant): the
blog's printed worked example, the Sylvester recursion, self-inverse and
norm, closed forms, exactness of the rotation sum for fp16 inputs against
rational arithmetic, invariance of exact attention under the rotation, and
the rotated cache's attention against torch's float64 SDPA on the dequantised
rotated rows with the inverse rotation done by scipy's Hadamard matrix."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import kvq_synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hadamard_example.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, *vals = line.split()
        rows[name] = np.array([float(v) for v in vals])
    return rows


def test_printed_example(oracle_mod):
    g = _golden()
    y = oracle_mod.hadamard(g["original"])
    assert np.array_equal(np.round(y, 3), g["rotated"])
    assert np.allclose(oracle_mod.hadamard(y), g["recovered"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [2, 4, 8, 32, 128, 256])
def test_sylvester_recursion(oracle_mod, n):
    # H_n [u; v] / sqrt(n) = [H_m (u + v); H_m (u - v)] / sqrt(n), m = n / 2
    x = kvq_synth.normal((3, n), [90, n, 0]).astype(np.float64)
    u, v = x[:, : n // 2], x[:, n // 2:]
    m = n // 2
    hu, hv = oracle_mod.hadamard(u) * math.sqrt(m), oracle_mod.hadamard(v) * math.sqrt(m)
    want = np.concatenate([hu + hv, hu - hv], axis=1) / math.sqrt(n)
    assert np.allclose(oracle_mod.hadamard(x), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [1, 4, 64, 128, 256])
def test_self_inverse_and_norm(oracle_mod, n):
    x = kvq_synth.normal((5, n), [91, n, 0]).astype(np.float64)
    y = oracle_mod.hadamard(x)
    assert np.allclose(oracle_mod.hadamard(y), x, rtol=0, atol=1e-13)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


@pytest.mark.parametrize("n", [4, 128])
def test_closed_forms(oracle_mod, n):
    e0 = np.zeros(n)
    e0[0] = 1.0
    assert np.allclose(oracle_mod.hadamard(e0), np.full(n, 1 / math.sqrt(n)), rtol=0, atol=1e-15)
    const = np.full(n, 0.75)
    want = np.zeros(n)
    want[0] = 0.75 * math.sqrt(n)
    assert np.allclose(oracle_mod.hadamard(const), want, rtol=0, atol=1e-13)


def test_non_power_of_two_rejected(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.hadamard(np.zeros(12))


def _exact_rotation(x16, n):
    """fl64(S * c), S the exact rational sum, c = 1.0 / sqrt(n) in IEEE
    float64 (correctly rounded sqrt and division, as the oracle)."""
    c = Fraction(1.0 / math.sqrt(n))
    out = []
    for i in range(n):
        s = Fraction(0)
        for j in range(n):
            t = Fraction(float(x16[j]))
            s += -t if bin(i & j).count("1") % 2 else t
        out.append(float(s * c))
    return np.array(out)


@pytest.mark.parametrize("n", [64, 128])
def test_rotation_sum_exact_for_fp16(oracle_mod, n):
    # widest spread an fp16 row can have: subnormals next to values near 65504
    rng = np.random.default_rng(92)
    bits = rng.integers(0, 0x7BFF, size=(6, n), dtype=np.int64).astype(np.uint16)
    bits |= (rng.integers(0, 2, size=(6, n)) << 15).astype(np.uint16)
    x = bits.view(np.float16)
    x[0, :8] = np.array([6e-8, -6e-8, 65504, -65504, 1e-7, 3.0, -2.0**-24, 2.0**-14], dtype=np.float16)
    y = oracle_mod.hadamard(x)
    for r in range(x.shape[0]):
        assert np.array_equal(y[r], _exact_rotation(x[r], n))


def test_exact_attention_is_rotation_invariant(oracle_mod):
    # softmax(a q.K^T) V computed directly equals the rotated computation
    # rotated back, in float64 (no quantisation)
    d, s = 128, 300
    q = kvq_synth.normal((4, d), [93, 0]).astype(np.float64)
    k = kvq_synth.normal((s, d), [93, 1]).astype(np.float64)
    v = kvq_synth.normal((s, d), [93, 2]).astype(np.float64)
    a = 1 / math.sqrt(d)

    def attend(q, k, v):
        sc = a * q @ k.T
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        return (w @ v) / w.sum(axis=1, keepdims=True)

    direct = attend(q, k, v)
    rotated = oracle_mod.hadamard(attend(oracle_mod.hadamard(q), oracle_mod.hadamard(k), oracle_mod.hadamard(v)))
    assert np.allclose(rotated, direct, rtol=0, atol=1e-12)


def test_rotated_cache_attention_matches_torch(oracle_mod):
    hq, hkv, d, s = 8, 2, 128, 700
    q = kvq_synth.to_f16(kvq_synth.normal((1, hq, d), [94, 0]))
    k = kvq_synth.to_f16(kvq_synth.normal((1, hkv, s, d), [94, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, hkv, s, d), [94, 2]))
    c = oracle_mod.Cache(1, hkv, d, s, 64)
    c.append_rotated(k, v, 0)
    got = oracle_mod.sdpa_rotated(c, s, q, 1 / math.sqrt(d))
    kd = oracle_mod.dequantize_rows(c.k_q, c.k_scale, c.k_bias, 64)
    vd = oracle_mod.dequantize_rows(c.v_q, c.v_scale, c.v_bias, 64)
    hn = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)
    qr = torch.from_numpy(q.astype(np.float64) @ hn.T)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qr, torch.from_numpy(kd), torch.from_numpy(vd),
                                                         scale=1 / math.sqrt(d), enable_gqa=True)
    want = o[:, :, 0, :].numpy() @ hn.T
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_rotated_append_quantises_rotated_rows(oracle_mod):
    k = kvq_synth.to_f16(kvq_synth.normal((1, 2, 5, 128), [95, 0]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, 2, 5, 128), [95, 1]))
    c = oracle_mod.Cache(1, 2, 128, 8, 64)
    c.append_rotated(k, v, 2)
    w, sc, bi = oracle_mod.quantize_rows(oracle_mod.hadamard(k).astype(np.float32), 64)
    assert np.array_equal(c.k_q[:, :, 2:7], w) and np.array_equal(c.k_scale[:, :, 2:7], sc)
    assert np.array_equal(c.k_bias[:, :, 2:7], bi)
    assert not c.k_q[:, :, :2].any() and not c.k_q[:, :, 7:].any()
    with pytest.raises(TypeError):
        c.append_rotated(k.astype(np.float32), v, 0)


def test_rotation_lowers_error_on_outlier_keys(oracle_mod):
    # the rotation spreads outlier channels, so the quantisation error of the
    # rows (measured after rotating back) drops: the method's stated purpose
    _, k, _, _ = kvq_synth.outlier_kv(total=512)
    rows = k[0, :, :256].reshape(-1, 128)
    plain = oracle_mod.dequantize_rows(*oracle_mod.quantize_rows(rows, 64), 64)
    rot = oracle_mod.hadamard(oracle_mod.dequantize_rows(
        *oracle_mod.quantize_rows(oracle_mod.hadamard(rows).astype(np.float32), 64), 64))
    x = rows.astype(np.float64)
    e_plain = np.linalg.norm(plain - x) / np.linalg.norm(x)
    e_rot = np.linalg.norm(rot - x) / np.linalg.norm(x)
    assert e_rot < 0.5 * e_plain, (e_rot, e_plain)

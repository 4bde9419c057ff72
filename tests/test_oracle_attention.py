"""Pins for the oracle's decode attention over the quantised cache: a library
routine on the dequantised values (torch's float64 SDPA, GQA included),
closed forms and invariants."""

import numpy as np
import pytest
import torch

import kvq_synth


def _cache(oracle_mod, k, v, cap=None, G=64):
    B, Hkv, S, D = k.shape
    c = oracle_mod.Cache(B, Hkv, D, cap or S, G)
    c.append(k, v, 0)
    return c


def _deq(oracle_mod, c, S):
    kd = oracle_mod.dequantize_rows(c.k_q[:, :, :S], c.k_scale[:, :, :S], c.k_bias[:, :, :S], c.G)
    vd = oracle_mod.dequantize_rows(c.v_q[:, :, :S], c.v_scale[:, :, :S], c.v_bias[:, :, :S], c.G)
    return kd, vd


def _torch_ref(q, kd, vd, alpha):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[:, :, None, :]  # [B,Hq,1,D]
    kt = torch.from_numpy(kd)
    vt = torch.from_numpy(vd)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=alpha,
                                                         enable_gqa=kt.shape[1] != qt.shape[1])
    return o[:, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,d,s,alpha", [(8, 2, 128, 1024, 1 / np.sqrt(128)), (4, 4, 64, 37, 0.3),
                                              (8, 1, 256, 300, 1.0), (6, 2, 64, 1, 0.125)])
def test_matches_torch_sdpa_on_dequantised(oracle_mod, hq, hkv, d, s, alpha):
    q = kvq_synth.normal((1, hq, d), [50, hq, d, s, 0])
    k = kvq_synth.normal((1, hkv, s, d), [50, hq, d, s, 1])
    v = kvq_synth.normal((1, hkv, s, d), [50, hq, d, s, 2])
    c = _cache(oracle_mod, k, v)
    kd, vd = _deq(oracle_mod, c, s)
    got = oracle_mod.sdpa(c, s, q, alpha)
    ref = _torch_ref(q, kd, vd, alpha)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_batch_two(oracle_mod):
    q = kvq_synth.normal((2, 4, 64), [51, 0])
    k = kvq_synth.normal((2, 2, 50, 64), [51, 1])
    v = kvq_synth.normal((2, 2, 50, 64), [51, 2])
    c = _cache(oracle_mod, k, v, cap=64)
    kd, vd = _deq(oracle_mod, c, 50)
    np.testing.assert_allclose(oracle_mod.sdpa(c, 50, q, 0.2), _torch_ref(q, kd, vd, 0.2), rtol=1e-12, atol=1e-13)


def test_constant_v_gives_that_row(oracle_mod):
    k = kvq_synth.normal((1, 2, 700, 128), [52, 1])
    row = kvq_synth.normal((128,), [52, 2]).astype(np.float16)
    v = np.broadcast_to(row, (1, 2, 700, 128)).copy()
    q = kvq_synth.normal((1, 8, 128), [52, 0])
    c = _cache(oracle_mod, k, v)
    got = oracle_mod.sdpa(c, 700, q, 1.0)
    vrow = oracle_mod.dequantize_rows(c.v_q[0, 0, :1], c.v_scale[0, 0, :1], c.v_bias[0, 0, :1])[0]
    np.testing.assert_allclose(got, np.broadcast_to(vrow, got.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("tstar", [0, 511, 512, 1199])
def test_one_hot_score_selects_row(oracle_mod, tstar):
    S, D = 1200, 128
    k = np.zeros((1, 1, S, D), dtype=np.float32)
    k[0, 0, tstar] = 8.0
    v = kvq_synth.normal((1, 1, S, D), [53, 1])
    q = np.full((1, 2, D), 8.0, dtype=np.float32)
    c = _cache(oracle_mod, k, v)
    got = oracle_mod.sdpa(c, S, q, 1.0)
    _, vd = _deq(oracle_mod, c, S)
    np.testing.assert_array_equal(got[0, 0], vd[0, 0, tstar])
    np.testing.assert_array_equal(got[0, 1], vd[0, 0, tstar])


def test_zero_query_gives_mean(oracle_mod):
    k = kvq_synth.normal((1, 2, 333, 64), [54, 1])
    v = kvq_synth.normal((1, 2, 333, 64), [54, 2])
    c = _cache(oracle_mod, k, v)
    got = oracle_mod.sdpa(c, 333, np.zeros((1, 4, 64)), 0.7)
    _, vd = _deq(oracle_mod, c, 333)
    mean = vd.mean(axis=2)  # [1,2,64]
    np.testing.assert_allclose(got, np.repeat(mean, 2, axis=1), rtol=1e-13, atol=1e-14)


def test_single_row(oracle_mod):
    k = kvq_synth.normal((1, 1, 1, 128), [55, 1])
    v = kvq_synth.normal((1, 1, 1, 128), [55, 2])
    c = _cache(oracle_mod, k, v, cap=8)
    _, vd = _deq(oracle_mod, c, 1)
    got = oracle_mod.sdpa(c, 1, kvq_synth.normal((1, 3, 128), [55, 0]), 5.0)
    for h in range(3):
        np.testing.assert_array_equal(got[0, h], vd[0, 0, 0])


def test_two_rows_sigmoid(oracle_mod):
    k = kvq_synth.normal((1, 1, 2, 64), [56, 1])
    v = kvq_synth.normal((1, 1, 2, 64), [56, 2])
    q = kvq_synth.normal((1, 1, 64), [56, 0]).astype(np.float64)
    c = _cache(oracle_mod, k, v)
    kd, vd = _deq(oracle_mod, c, 2)
    a = 0.4
    s0, s1 = a * q[0, 0] @ kd[0, 0, 0], a * q[0, 0] @ kd[0, 0, 1]
    sig = 1.0 / (1.0 + np.exp(-(s0 - s1)))
    ref = sig * vd[0, 0, 0] + (1 - sig) * vd[0, 0, 1]
    np.testing.assert_allclose(oracle_mod.sdpa(c, 2, q, a)[0, 0], ref, rtol=1e-13, atol=1e-14)


def test_row_permutation_invariance(oracle_mod):
    S = 400
    k = kvq_synth.normal((1, 2, S, 128), [57, 1])
    v = kvq_synth.normal((1, 2, S, 128), [57, 2])
    q = kvq_synth.normal((1, 4, 128), [57, 0])
    c = _cache(oracle_mod, k, v)
    perm = np.random.default_rng(5).permutation(S)
    c2 = _cache(oracle_mod, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(oracle_mod.sdpa(c, S, q, 0.09), oracle_mod.sdpa(c2, S, q, 0.09),
                               rtol=1e-12, atol=1e-14)


def test_prefix_only(oracle_mod):
    """Rows at or beyond skv are ignored (the cache may hold more capacity)."""
    k = kvq_synth.normal((1, 2, 300, 64), [58, 1])
    v = kvq_synth.normal((1, 2, 300, 64), [58, 2])
    q = kvq_synth.normal((1, 2, 64), [58, 0])
    c_full = _cache(oracle_mod, k, v)
    c_pre = _cache(oracle_mod, k[:, :, :200], v[:, :, :200], cap=300)
    np.testing.assert_array_equal(oracle_mod.sdpa(c_full, 200, q, 0.5), oracle_mod.sdpa(c_pre, 200, q, 0.5))


@pytest.mark.parametrize("chunk", [1, 7, 64, 512, 1000, 1031])
def test_partials_combine_to_full(oracle_mod, chunk):
    S = 1000
    k = kvq_synth.normal((1, 2, S, 128), [59, 1])
    v = kvq_synth.normal((1, 2, S, 128), [59, 2])
    q = kvq_synth.normal((1, 8, 128), [59, 0])
    c = _cache(oracle_mod, k, v)
    m, l, acc = oracle_mod.sdpa_partials(c, S, q, 1 / np.sqrt(128), chunk)
    nc = (S + chunk - 1) // chunk
    assert m.shape == (1, 8, nc) and acc.shape == (1, 8, nc, 128)
    lens = np.minimum(chunk, S - chunk * np.arange(nc))
    assert np.all(l >= 1.0) and np.all(l <= lens[None, None, :] + 1e-9)
    full = oracle_mod.sdpa(c, S, q, 1 / np.sqrt(128))
    np.testing.assert_allclose(oracle_mod.combine_partials(m, l, acc), full, rtol=1e-12, atol=1e-14)


def test_partial_is_attention_over_its_chunk(oracle_mod):
    """acc_c / l_c is attention restricted to chunk c, and m_c is the largest
    score in it (checked against torch on the dequantised chunk)."""
    S, chunk = 700, 256
    k = kvq_synth.normal((1, 1, S, 64), [60, 1])
    v = kvq_synth.normal((1, 1, S, 64), [60, 2])
    q = kvq_synth.normal((1, 2, 64), [60, 0])
    c = _cache(oracle_mod, k, v)
    kd, vd = _deq(oracle_mod, c, S)
    m, l, acc = oracle_mod.sdpa_partials(c, S, q, 0.3, chunk)
    for ci in range(3):
        sl = slice(ci * chunk, min(S, (ci + 1) * chunk))
        ref = _torch_ref(q, kd[:, :, sl], vd[:, :, sl], 0.3)
        np.testing.assert_allclose(acc[:, :, ci] / l[:, :, ci, None], ref, rtol=1e-12, atol=1e-14)
        scores = 0.3 * np.einsum("bhd,bhtd->bht", q.astype(np.float64), kd[:, 0:1, sl].repeat(2, axis=1))
        np.testing.assert_allclose(m[:, :, ci], scores.max(axis=2), rtol=1e-13)

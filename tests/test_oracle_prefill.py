"""Pins for the oracle's prefill-side attention (Sq > 1 query positions over
the quantised cache, causal): torch's float64 SDPA with the causal mask
shifted by the prefix length on the dequantised cache (GQA included), the
causal invariance (rows after a query's position do not change its output),
and the reductions Sq = 1 (the decode attention) and full visibility of the
prefix."""

import numpy as np
import pytest
import torch

import kvq_synth


def _deq(oracle_mod, c, S):
    kd = oracle_mod.dequantize_rows(c.k_q[:, :, :S], c.k_scale[:, :, :S], c.k_bias[:, :, :S], c.G, c.bits)
    vd = oracle_mod.dequantize_rows(c.v_q[:, :, :S], c.v_scale[:, :, :S], c.v_bias[:, :, :S], c.G, c.bits)
    return kd, vd


def _torch_causal(q, kd, vd, alpha, q_start):
    """torch float64 SDPA, query i of the block at absolute position
    q_start + i seeing rows t <= q_start + i."""
    B, Hq, Sq, D = q.shape
    S = kd.shape[2]
    mask = np.arange(S)[None, :] <= (q_start + np.arange(Sq))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(q, dtype=np.float64)), torch.from_numpy(kd), torch.from_numpy(vd),
        attn_mask=torch.from_numpy(mask), scale=alpha, enable_gqa=kd.shape[1] != Hq)
    return o.numpy()


@pytest.mark.parametrize("hq,hkv,d,q_start,sq,alpha,bits", [(8, 2, 128, 0, 37, 1 / np.sqrt(128), 4),
                                                            (8, 2, 128, 500, 64, 1 / np.sqrt(128), 4),
                                                            (4, 4, 64, 13, 20, 0.3, 4),
                                                            (16, 1, 256, 100, 9, 1.0, 4),
                                                            (8, 2, 128, 300, 33, 1 / np.sqrt(128), 8)])
def test_matches_torch_causal_sdpa(oracle_mod, hq, hkv, d, q_start, sq, alpha, bits):
    S = q_start + sq
    q = kvq_synth.normal((1, hq, sq, d), [60, hq, d, q_start, 0])
    k = kvq_synth.normal((1, hkv, S, d), [60, hq, d, q_start, 1])
    v = kvq_synth.normal((1, hkv, S, d), [60, hq, d, q_start, 2])
    c = oracle_mod.Cache(1, hkv, d, S + 5, 64 if d >= 64 else d, bits=bits)
    c.append(k, v, 0)
    kd, vd = _deq(oracle_mod, c, S)
    got = oracle_mod.sdpa_prefill(c, q_start, q, alpha)
    np.testing.assert_allclose(got, _torch_causal(q, kd, vd, alpha, q_start), rtol=1e-12, atol=1e-13)


def test_causal_rows_do_not_leak(oracle_mod):
    """Changing cache rows after a query's position leaves that query's
    output unchanged, and changes the outputs of later queries."""
    q_start, sq, S = 40, 16, 56
    q = kvq_synth.normal((1, 8, sq, 128), [61, 0])
    k = kvq_synth.normal((1, 2, S, 128), [61, 1])
    v = kvq_synth.normal((1, 2, S, 128), [61, 2])
    c1 = oracle_mod.Cache(1, 2, 128, S, 64)
    c1.append(k, v, 0)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 50:] += 3.0
    v2[:, :, 50:] -= 2.0
    c2 = oracle_mod.Cache(1, 2, 128, S, 64)
    c2.append(k2, v2, 0)
    o1 = oracle_mod.sdpa_prefill(c1, q_start, q, 0.1)
    o2 = oracle_mod.sdpa_prefill(c2, q_start, q, 0.1)
    np.testing.assert_array_equal(o1[:, :, :10], o2[:, :, :10])   # positions 40..49
    assert np.abs(o1[:, :, 10:] - o2[:, :, 10:]).min() > 0        # positions 50..55 see the change


def test_single_position_is_decode(oracle_mod):
    q = kvq_synth.normal((1, 8, 1, 128), [62, 0])
    k = kvq_synth.normal((1, 2, 300, 128), [62, 1])
    v = kvq_synth.normal((1, 2, 300, 128), [62, 2])
    c = oracle_mod.Cache(1, 2, 128, 300, 64)
    c.append(k, v, 0)
    got = oracle_mod.sdpa_prefill(c, 299, q, 0.2)
    np.testing.assert_array_equal(got[:, :, 0], oracle_mod.sdpa(c, 300, q[:, :, 0], 0.2))


def test_first_position_sees_one_row(oracle_mod):
    """With no prefix the first query sees only row 0: its output is that
    row's dequantised V (softmax over one score is 1)."""
    q = kvq_synth.normal((1, 4, 5, 64), [63, 0])
    k = kvq_synth.normal((1, 1, 5, 64), [63, 1])
    v = kvq_synth.normal((1, 1, 5, 64), [63, 2])
    c = oracle_mod.Cache(1, 1, 64, 5, 64)
    c.append(k, v, 0)
    got = oracle_mod.sdpa_prefill(c, 0, q, 1.0)
    _, vd = _deq(oracle_mod, c, 5)
    for h in range(4):
        np.testing.assert_allclose(got[0, h, 0], vd[0, 0, 0], rtol=0, atol=1e-15)

"""GPU parity of prefill-side attention over the quantised cache, int4 and
8-bit codes (kvq_sdpa_int4_prefill: Sq > 1 query positions, causal, against
the float64 oracle's sdpa_prefill on the same packed cache)."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import check_attention, gpu_cache_from_oracle, note, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4  # the matrix-core gate of the decode tests


def _case(B, hq, hkv, q_start, sq, seed, alpha=None, cap=None, bits=4, D=128):
    S = q_start + sq
    q = kvq_synth.normal((B, hq, sq, D), [90, seed, 0]).astype(np.float16)
    k = kvq_synth.normal((B, hkv, S, D), [90, seed, 1]).astype(np.float16)
    v = kvq_synth.normal((B, hkv, S, D), [90, seed, 2]).astype(np.float16)
    oc = oracle.Cache(B, hkv, D, cap or S, 64, bits=bits)
    oc.append(k, v, 0)
    return q, oc, (1 / np.sqrt(D) if alpha is None else alpha)


def _run(oc, q_start, q, alpha):
    gc = gpu_cache_from_oracle(oc)
    out = kvq.sdpa_int4_prefill(gc, q_start, to_dev(q), alpha)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("q_start,sq", [(0, 1), (0, 2), (0, 7), (0, 33), (5, 64), (511, 100), (1000, 17),
                                        (31, 1), (32, 32), (4000, 96)])
def test_gqa4(q_start, sq):
    note("prefill gqa4 q_start=%d sq=%d" % (q_start, sq))
    q, oc, alpha = _case(1, 8, 2, q_start, sq, seed=q_start * 1000 + sq)
    got = _run(oc, q_start, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, q_start, q, alpha), REL_L2, label="prefill")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 16), (16, 1), (6, 2), (12, 4)])
def test_head_layouts(hq, hkv):
    """GQA 8 (the Llama layer), MHA, 16 heads per KV head, and ratios that do
    not divide the 32 query columns of a wavefront (3, with a position split
    between the wavefront's two 16-column blocks)."""
    note("prefill heads hq=%d hkv=%d" % (hq, hkv))
    q, oc, alpha = _case(1, hq, hkv, 300, 45, seed=hq * 100 + hkv)
    got = _run(oc, 300, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 300, q, alpha), REL_L2, label="prefill heads")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("hq,hkv,q32", [(64, 2, False), (40, 2, False), (32, 1, True), (24, 1, False)])
def test_wide_gqa(hq, hkv, q32, bits):
    """More than 16 query heads per KV head at D 128: each wavefront takes one
    position of all the KV head's query heads (32 and 20 of its 32 columns,
    with an fp32 query too)."""
    note("prefill wide gqa hq=%d hkv=%d q32=%d bits=%d" % (hq, hkv, q32, bits))
    q, oc, alpha = _case(1, hq, hkv, 700, 37, seed=hq * 10 + hkv + bits, bits=bits)
    if q32:
        q = (q.astype(np.float32) + kvq_synth.normal(q.shape, [91, hq]).astype(np.float32) * 1e-3)
    got = _run(oc, 700, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 700, q, alpha), REL_L2, label="prefill wide gqa")


@pytest.mark.parametrize("bits,D", [(4, 128), (8, 128), (4, 256), (8, 256)])
def test_batch_two_and_spare_capacity(bits, D):
    note("prefill batch 2 bits=%d D=%d" % (bits, D))
    q, oc, alpha = _case(2, 8, 2, 200, 40, seed=7 + bits + D, cap=400, bits=bits, D=D)
    got = _run(oc, 200, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 200, q, alpha), REL_L2, label="prefill batch")


def test_unscaled_scores():
    """Softmax scale 1 on N(0,1) rows: scores of O(10), weights far from flat."""
    note("prefill alpha 1")
    q, oc, alpha = _case(1, 8, 2, 700, 20, seed=11, alpha=1.0)
    got = _run(oc, 700, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 700, q, alpha), REL_L2, atol=1e-3, rtol=1e-3, label="prefill a1")


def test_first_position_is_row_zero():
    note("prefill first row")
    q, oc, alpha = _case(1, 8, 2, 0, 3, seed=12)
    got = _run(oc, 0, q, alpha)
    vd = oracle.dequantize_rows(oc.v_q[:, :, :1], oc.v_scale[:, :, :1], oc.v_bias[:, :, :1], 64)
    for h in range(8):
        np.testing.assert_allclose(got[0, h, 0], vd[0, h // 4, 0], rtol=1e-5, atol=1e-6)


def test_outlier_chunked_prefill_sampled():
    """The outlier workload's append: 4096 new rows per KV head at row 61440
    (quantised by the GPU append), then prefill attention for those 4096
    positions; sampled positions (first, second, middle, last) checked against
    the oracle on all heads."""
    note("prefill outlier 4096 at 61440")
    total, prefix = 65536, 61440
    _, k, v, _ = kvq_synth.outlier_kv(total)
    q = kvq_synth.normal((1, 64, total - prefix, 128), [91, 0]).astype(np.float16)
    alpha = 1 / np.sqrt(128)
    oc = oracle.Cache(1, 8, 128, total, 64)
    oc.append(k[:, :, :prefix], v[:, :, :prefix], 0)
    gc = gpu_cache_from_oracle(oc)
    kvq.quantize_kv_append(gc, prefix, to_dev(np.ascontiguousarray(k[:, :, prefix:])),
                           to_dev(np.ascontiguousarray(v[:, :, prefix:])))
    out = kvq.sdpa_int4_prefill(gc, prefix, to_dev(q), alpha)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    oc.append(k[:, :, prefix:], v[:, :, prefix:], prefix)
    for i in (0, 1, 2047, 4095):
        ref = oracle.sdpa(oc, prefix + i + 1, np.ascontiguousarray(q[:, :, i]), alpha)
        check_attention(got[:, :, i], ref, REL_L2, label="prefill outlier pos %d" % i)


@pytest.mark.parametrize("q_start,sq", [(0, 1), (0, 33), (5, 64), (511, 100), (4000, 96)])
def test_int8_gqa4(q_start, sq):
    """8-bit codes: the same positions and prefixes as the int4 cases."""
    note("prefill int8 gqa4 q_start=%d sq=%d" % (q_start, sq))
    q, oc, alpha = _case(1, 8, 2, q_start, sq, seed=7000 + q_start * 1000 + sq, bits=8)
    got = _run(oc, q_start, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, q_start, q, alpha), REL_L2, label="prefill int8")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 16), (16, 1), (6, 2)])
def test_int8_head_layouts(hq, hkv):
    note("prefill int8 heads hq=%d hkv=%d" % (hq, hkv))
    q, oc, alpha = _case(1, hq, hkv, 300, 45, seed=8000 + hq * 100 + hkv, bits=8)
    got = _run(oc, 300, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 300, q, alpha), REL_L2, label="prefill int8 heads")


def test_int8_unscaled_scores():
    note("prefill int8 alpha 1")
    q, oc, alpha = _case(1, 8, 2, 700, 20, seed=8011, alpha=1.0, bits=8)
    got = _run(oc, 700, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 700, q, alpha), REL_L2, atol=1e-3, rtol=1e-3, label="prefill int8 a1")


def test_int8_outlier_chunked_prefill_sampled():
    """The outlier workload's 4096-row append into an 8-bit cache (GPU append),
    then prefill attention for those positions, sampled on all heads."""
    note("prefill int8 outlier 4096 at 61440")
    total, prefix = 65536, 61440
    _, k, v, _ = kvq_synth.outlier_kv(total)
    q = kvq_synth.normal((1, 64, total - prefix, 128), [91, 1]).astype(np.float16)
    alpha = 1 / np.sqrt(128)
    oc = oracle.Cache(1, 8, 128, total, 64, bits=8)
    oc.append(k[:, :, :prefix], v[:, :, :prefix], 0)
    gc = gpu_cache_from_oracle(oc)
    kvq.quantize_kv_append(gc, prefix, to_dev(np.ascontiguousarray(k[:, :, prefix:])),
                           to_dev(np.ascontiguousarray(v[:, :, prefix:])))
    out = kvq.sdpa_int4_prefill(gc, prefix, to_dev(q), alpha)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    oc.append(k[:, :, prefix:], v[:, :, prefix:], prefix)
    for i in (0, 1, 2047, 4095):
        ref = oracle.sdpa(oc, prefix + i + 1, np.ascontiguousarray(q[:, :, i]), alpha)
        check_attention(got[:, :, i], ref, REL_L2, label="prefill int8 outlier pos %d" % i)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("q_start,sq", [(0, 33), (511, 100)])
def test_fp32_queries(bits, q_start, sq):
    """fp32 queries (hi + lo fp16 halves) against the oracle on the same fp32 values."""
    note("prefill fp32 q bits=%d q_start=%d sq=%d" % (bits, q_start, sq))
    q16, oc, alpha = _case(1, 8, 2, q_start, sq, seed=9000 + bits * 100 + sq, bits=bits)
    q = (q16.astype(np.float32) * np.float32(1.0 + 2.0 ** -13)).astype(np.float32)  # not fp16-exact
    gc = gpu_cache_from_oracle(oc)
    got = kvq.sdpa_int4_prefill(gc, q_start, to_dev(q), alpha)
    torch.cuda.synchronize()
    check_attention(got.cpu().numpy(), oracle.sdpa_prefill(oc, q_start, q, alpha), REL_L2, label="prefill fp32 q")


@pytest.mark.parametrize("bits", [4, 8])
def test_rotated_cache_prefill(bits):
    """Prefill over a Hadamard-rotated cache from the entry points: rotate q
    (fp32), prefill with fp32 queries, rotate the output back; against the
    oracle's rotated attention, position by position."""
    note("prefill on a rotated cache bits=%d" % bits)
    q_start, sq, hq, hkv = 700, 24, 8, 2
    S = q_start + sq
    q = kvq_synth.normal((1, hq, sq, 128), [92, bits, 0]).astype(np.float16)
    k = kvq_synth.normal((1, hkv, S, 128), [92, bits, 1]).astype(np.float16)
    v = kvq_synth.normal((1, hkv, S, 128), [92, bits, 2]).astype(np.float16)
    alpha = 1 / np.sqrt(128)
    oc = oracle.Cache(1, hkv, 128, S, 64, bits=bits)
    oc.append_rotated(k, v, 0)
    gc = gpu_cache_from_oracle(oc)
    qr = kvq.hadamard_rotate(to_dev(q))
    out = kvq.sdpa_int4_prefill(gc, q_start, qr, alpha)
    kvq.hadamard_rotate(out, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i in range(sq):
        ref = oracle.sdpa_rotated(oc, q_start + i + 1, np.ascontiguousarray(q[:, :, i]), alpha)
        check_attention(got[:, :, i], ref, REL_L2, label="rotated prefill pos %d" % i)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("q_start,sq", [(0, 1), (0, 33), (423, 40), (1000, 17)])
def test_head_dim_256(bits, q_start, sq):
    """D = 256 (four scale groups, two sets of value words): the Gemma-style
    layer of the decode tests, 32 query heads on 16 KV heads, alpha 1."""
    note("prefill D256 bits=%d q_start=%d sq=%d" % (bits, q_start, sq))
    q, oc, _ = _case(1, 32, 16, q_start, sq, seed=9500 + bits * 100 + sq, bits=bits, D=256)
    q = (q.astype(np.float32) * np.float32(0.25)).astype(np.float16)  # O(10) scores at alpha 1
    got = _run(oc, q_start, q, 1.0)
    check_attention(got, oracle.sdpa_prefill(oc, q_start, q, 1.0), REL_L2, atol=1e-3, rtol=1e-3,
                    label="prefill D256")


def test_head_dim_256_fp32_queries_and_gqa8():
    note("prefill D256 fp32 q, 8 heads per KV head")
    q16, oc, alpha = _case(1, 16, 2, 300, 45, seed=9600, D=256)
    q = (q16.astype(np.float32) * np.float32(1.0 + 2.0 ** -13)).astype(np.float32)
    gc = gpu_cache_from_oracle(oc)
    got = kvq.sdpa_int4_prefill(gc, 300, to_dev(q), alpha)
    torch.cuda.synchronize()
    check_attention(got.cpu().numpy(), oracle.sdpa_prefill(oc, 300, q, alpha), REL_L2, label="prefill D256 fp32")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("q_start,sq", [(0, 1), (0, 33), (300, 45), (1000, 17), (4000, 96)])
def test_head_dim_64(bits, q_start, sq):
    """D = 64 (one scale group; each value column half a word): 32 query
    heads on 8 KV heads."""
    note("prefill D64 bits=%d q_start=%d sq=%d" % (bits, q_start, sq))
    q, oc, alpha = _case(1, 32, 8, q_start, sq, seed=9700 + bits * 100 + sq, bits=bits, D=64)
    got = _run(oc, q_start, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, q_start, q, alpha), REL_L2, label="prefill D64")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("hq,hkv,q32", [(16, 16, False), (64, 2, True), (12, 4, False), (8, 2, True)])
def test_head_dim_64_layouts(bits, hq, hkv, q32):
    """D = 64: multi-head, 32 heads per KV head (one position per
    wavefront), GQA 3, and fp32 queries."""
    note("prefill D64 hq=%d hkv=%d q32=%d bits=%d" % (hq, hkv, q32, bits))
    q, oc, alpha = _case(1, hq, hkv, 500, 40, seed=9800 + hq * 10 + hkv + bits, bits=bits, D=64)
    if q32:
        q = (q.astype(np.float32) + kvq_synth.normal(q.shape, [92, hq]).astype(np.float32) * 1e-3)
    got = _run(oc, 500, q, alpha)
    check_attention(got, oracle.sdpa_prefill(oc, 500, q, alpha), REL_L2, label="prefill D64 layouts")


def test_head_dim_64_unscaled_batch_two():
    note("prefill D64 alpha 1, batch 2")
    q, oc, _ = _case(2, 8, 2, 250, 30, seed=9900, cap=301, D=64)
    q = (q.astype(np.float32) * np.float32(0.5)).astype(np.float16)
    got = _run(oc, 250, q, 1.0)
    check_attention(got, oracle.sdpa_prefill(oc, 250, q, 1.0), REL_L2, atol=1e-3, rtol=1e-3, label="prefill D64 a1")


@pytest.mark.parametrize("what", ["g32", "d64_g32"])
def test_unsupported_shapes_refused(what):
    note("prefill refuses %s" % what)
    D = 64 if what == "d64_g32" else 128
    G = 32
    bits = 4
    gc = kvq.QuantKVCache(1, 2, D, 64, G, device="cuda", bits=bits)
    q = torch.zeros((1, 8, 4, D), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.sdpa_int4_prefill(gc, 10, q, 0.1)
    assert e.value.status == -7


def test_prompt_from_row_zero_sampled():
    """A 1200-position prompt from row 0 on the Llama layer's heads: many
    workgroups, a ragged last one, and the causal triangle; sampled positions
    (the first, tile and workgroup edges, the last) against the oracle's
    decode attention over the rows each position sees."""
    note("prefill prompt 1200 from row 0")
    sq, hq, hkv = 1200, 64, 8
    q = kvq_synth.normal((1, hq, sq, 128), [93, 0]).astype(np.float16)
    k = kvq_synth.normal((1, hkv, sq, 128), [93, 1]).astype(np.float16)
    v = kvq_synth.normal((1, hkv, sq, 128), [93, 2]).astype(np.float16)
    alpha = 1 / np.sqrt(128)
    oc = oracle.Cache(1, hkv, 128, sq, 64)
    oc.append(k, v, 0)
    got = _run(oc, 0, q, alpha)
    for i in (0, 1, 3, 4, 31, 32, 33, 599, 1023, 1024, 1199):
        ref = oracle.sdpa(oc, i + 1, np.ascontiguousarray(q[:, :, i]), alpha)
        check_attention(got[:, :, i], ref, REL_L2, label="prompt pos %d" % i)


@pytest.mark.parametrize("bits", [4, 8])
def test_small_value_ranges(bits):
    """V rows scaled by 2^-7 (int4 value scales near 2^-9, where the split of
    a scale into its top eight bits and the rest is still exact after
    halving) and K rows by 2^-4: the matrix-core products stay exact, so the
    usual gate holds."""
    note("prefill small value ranges bits=%d" % bits)
    q_start, sq, hq, hkv = 900, 40, 8, 2
    S = q_start + sq
    q = kvq_synth.normal((1, hq, sq, 128), [94, bits, 0]).astype(np.float16)
    k = (kvq_synth.normal((1, hkv, S, 128), [94, bits, 1]) * 2.0 ** -4).astype(np.float16)
    v = (kvq_synth.normal((1, hkv, S, 128), [94, bits, 2]) * 2.0 ** -7).astype(np.float16)
    alpha = 1 / np.sqrt(128)
    oc = oracle.Cache(1, hkv, 128, S, 64, bits=bits)
    oc.append(k, v, 0)
    got = _run(oc, q_start, q, alpha)
    ref = oracle.sdpa_prefill(oc, q_start, q, alpha)
    check_attention(got, ref, REL_L2, atol=2e-5, rtol=1e-2, label="prefill small values")


# 8-bit codes at D 128 with at most 16 query heads per KV head run in
# workgroups of four wavefronts of 16 query columns each (16 / n_rep
# positions per wavefront); above 16 heads, one wavefront of 32 columns.
# Cases: the boundary n_rep 16 / 20, and a last workgroup whose later
# wavefronts have no positions (n_rep 1: 64 positions per workgroup, sq 65
# and 130; n_rep 8: 8 positions per workgroup, sq 9), with fp32 queries.
@pytest.mark.parametrize("hq,hkv,q_start,sq,q32", [(16, 1, 0, 40, False), (20, 1, 0, 40, False),
                                                   (16, 1, 700, 9, True), (20, 1, 700, 9, True),
                                                   (2, 2, 0, 65, False), (4, 4, 300, 130, True),
                                                   (64, 8, 100, 9, False), (64, 8, 3000, 23, True)])
def test_int8_workgroup_edges(hq, hkv, q_start, sq, q32):
    note("prefill int8 workgroup edges hq=%d hkv=%d q_start=%d sq=%d q32=%d" % (hq, hkv, q_start, sq, q32))
    q, oc, alpha = _case(1, hq, hkv, q_start, sq, seed=77000 + hq * 100 + sq, bits=8)
    if q32:
        q = (q.astype(np.float32) * np.float32(1.0001)).astype(np.float32)
    check_attention(_run(oc, q_start, q, alpha), oracle.sdpa_prefill(oc, q_start, q, alpha), REL_L2,
                    label="int8 workgroup edges")

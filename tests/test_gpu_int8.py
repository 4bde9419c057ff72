"""GPU parity of the 8-bit cache (the Gemma page's "What I Tried" table lists
an int8 KV cache; the blog's decode driver takes 4 or 8 KV bits): the append
kernel must write the oracle's bytes bit for bit; the vector-ALU and the
one-wavefront matrix-core attention must match the float64 oracle on the
8-bit cache within the gates of the int4 tests; the other matrix-core
variants must refuse the format."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import (assert_cache_equal, canary_cache, check_attention, gpu_cache_from_oracle, note, run_sdpa,
                         to_dev)
from test_gpu_quantize import _append_and_check, _boundary_rows, _special_rows

pytestmark = pytest.mark.gpu

REL_L2 = 2e-5            # the vector-ALU gate of the int4 tests (fp32 throughout)
MFMA_REL_L2 = 1e-4       # the matrix-core gate of the int4 tests
REL_L2_UNSCALED = 1e-4   # softmax scale 1 (test_gpu_sdpa.py): score rounding passes undamped into the weights
KERNELS = [kvq.KERNEL_VALU, kvq.KERNEL_MFMA_WAVE, kvq.KERNEL_AUTO]
GATE = {kvq.KERNEL_VALU: REL_L2, kvq.KERNEL_MFMA_WAVE: MFMA_REL_L2, kvq.KERNEL_AUTO: MFMA_REL_L2}


def _run(gc, skv, q, alpha, kernel, chunk=512):
    """run_sdpa, skipping a forced one-wavefront run on a chunk it does not
    take (AUTO falls back to the vector-ALU kernel there)."""
    try:
        return run_sdpa(gc, skv, q, alpha, chunk=chunk, kernel=kernel)
    except kvq.KvqError as e:
        if kernel == kvq.KERNEL_MFMA_WAVE and e.status == -7:
            pytest.skip("chunk outside the one-wavefront kernel")
        raise


def _oracle_cache(k, v, cap=None, G=64):
    B, Hkv, S, D = k.shape
    oc = oracle.Cache(B, Hkv, D, cap or S, G, bits=8)
    oc.append(k, v, 0)
    return oc


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("B,Hkv,D,G,dt", [(2, 3, 64, 32, np.float32), (1, 2, 64, 64, np.float16),
                                          (1, 2, 128, 32, np.float16), (1, 2, 128, 128, np.float32),
                                          (2, 1, 256, 64, np.float16), (1, 3, 256, 128, np.float32)])
def test_append_shapes(B, Hkv, D, G, dt):
    note("int8 append B%d Hkv%d D%d G%d %s" % (B, Hkv, D, G, np.dtype(dt).name))
    k = kvq_synth.normal((B, Hkv, 77, D), [170, D, G, 1]).astype(dt)
    v = (3 * kvq_synth.normal((B, Hkv, 77, D), [170, D, G, 2])).astype(dt)
    _append_and_check(k, v, 5, 90, G, bits=8)


@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_append_special_values(dt):
    note("int8 append special values %s" % np.dtype(dt).name)
    x = _special_rows().astype(dt)
    _append_and_check(x[None, None], -x[None, None], 0, x.shape[0], bits=8)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_append_rounding_boundaries(G):
    """Quotients on and next to the 255 half-integers, where the reciprocal
    product can round differently from the correctly rounded quotient."""
    note("int8 append rounding boundaries G=%d" % G)
    x = _boundary_rows(G=G, L=255)
    _append_and_check(x[None, None], x[None, None, ::-1].copy(), 1, x.shape[0] + 2, G, bits=8)


def test_append_one_row_at_a_time():
    note("int8 append single rows")
    k = kvq_synth.to_f16(kvq_synth.normal((1, 8, 5, 128), [171, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, 8, 5, 128), [171, 2]))
    gc = canary_cache(1, 8, 128, 8, bits=8)
    for t in range(5):
        kvq.quantize_kv_append(gc, t, to_dev(np.ascontiguousarray(k[:, :, t:t + 1])),
                               to_dev(np.ascontiguousarray(v[:, :, t:t + 1])))
    torch.cuda.synchronize()
    oc = oracle.Cache(1, 8, 128, 8, bits=8)
    oc.append(k, v, 0)
    assert_cache_equal(gc, oc, slice(0, 5))


def test_append_llama_full_length():
    """The Llama-shaped layer at its longest context (131072 rows), fp16."""
    note("int8 append llama 1x8x131072x128 fp16")
    _, k, v, _ = kvq_synth.llama_layer(131072)
    gc = canary_cache(1, 8, 128, 131072, bits=8)
    kvq.quantize_kv_append(gc, 0, to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    oc = oracle.Cache(1, 8, 128, 131072, bits=8)
    oc.append(k, v, 0)
    assert_cache_equal(gc, oc)


# --------------------------------------------------------------- attention

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("skv,chunk", [(1, 512), (33, 512), (512, 512), (513, 512), (1000, 8), (1000, 64),
                                       (1000, 100), (1000, 3), (1500, 256), (1000, 2048)])
def test_ragged(kernel, skv, chunk):
    note("int8 sdpa ragged skv=%d chunk=%d kernel=%d" % (skv, chunk, kernel))
    q = kvq_synth.normal((1, 8, 128), [180, skv, 0]).astype(np.float16)
    k = kvq_synth.normal((1, 2, 1536, 128), [180, 1]).astype(np.float16)
    v = kvq_synth.normal((1, 2, 1536, 128), [180, 2]).astype(np.float16)
    oc = _oracle_cache(k, v)
    out, *_ = _run(gpu_cache_from_oracle(oc), skv, q, 0.0884, kernel, chunk=chunk)
    check_attention(out, oracle.sdpa(oc, skv, q, 0.0884), GATE[kernel], label="int8 ragged")


@pytest.mark.parametrize("B,Hq,Hkv,D,G,qdt", [(2, 4, 4, 64, 32, np.float32), (1, 6, 2, 128, 64, np.float16),
                                              (1, 16, 1, 128, 64, np.float16), (1, 8, 1, 256, 128, np.float32),
                                              (1, 2, 2, 256, 64, np.float16), (2, 8, 2, 128, 32, np.float32),
                                              (1, 4, 1, 64, 64, np.float16),
                                              # query heads of a KV head in blocks (32 -> 4 x 8, 20 -> 5 x 4)
                                              (1, 64, 2, 128, 64, np.float16), (1, 20, 1, 256, 128, np.float32)])
@pytest.mark.parametrize("kernel", KERNELS)
def test_shapes(kernel, B, Hq, Hkv, D, G, qdt):
    note("int8 sdpa shape B%d Hq%d Hkv%d D%d G%d kernel=%d" % (B, Hq, Hkv, D, G, kernel))
    S = 700
    q = kvq_synth.normal((B, Hq, D), [181, Hq, D, G, 0]).astype(qdt)
    k = kvq_synth.normal((B, Hkv, S, D), [181, Hq, D, G, 1]).astype(np.float16)
    v = kvq_synth.normal((B, Hkv, S, D), [181, Hq, D, G, 2]).astype(np.float16)
    oc = _oracle_cache(k, v, cap=S + 13, G=G)
    alpha = 1 / np.sqrt(D)
    try:
        out, *_ = run_sdpa(gpu_cache_from_oracle(oc), S, q, alpha, kernel=kernel)
    except kvq.KvqError as e:
        if kernel == kvq.KERNEL_MFMA_WAVE and e.status == -7:
            pytest.skip("shape outside the matrix-core kernels")  # D = 64
        raise
    check_attention(out, oracle.sdpa(oc, S, q, alpha), GATE[kernel], label="int8 shape")


def test_partials_match_oracle():
    note("int8 sdpa partials")
    q, k, v, alpha = kvq_synth.tiny_decode()
    oc = _oracle_cache(k, v)
    _, m, l, acc = run_sdpa(gpu_cache_from_oracle(oc), 1024, q, alpha, chunk=100, kernel=kvq.KERNEL_VALU)
    rm, rl, racc = oracle.sdpa_partials(oc, 1024, q, alpha, 100)
    np.testing.assert_allclose(m, rm, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(l, rl, rtol=1e-4)
    np.testing.assert_allclose(acc / l[..., None], racc / rl[..., None], rtol=1e-3, atol=1e-4)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("skv", [423, 4096])
def test_gemma_unscaled(kernel, skv):
    note("int8 sdpa gemma skv=%d kernel=%d" % (skv, kernel))
    q, k, v, alpha = kvq_synth.gemma_layer(skv)
    oc = _oracle_cache(k, v, cap=(skv + 7) // 8 * 8)
    out, *_ = _run(gpu_cache_from_oracle(oc), skv, q, alpha, kernel)
    check_attention(out, oracle.sdpa(oc, skv, q, alpha), REL_L2_UNSCALED, atol=1e-3, rtol=1e-3, label="int8 gemma")


@pytest.mark.parametrize("skv", [4096, 131072])
def test_llama_layer(skv):
    """The Llama layer, cache written by the GPU append, attention in the
    benchmark's launch configuration (chunk 512, automatic kernel choice);
    at 131072 rows two KV heads' query heads are checked."""
    note("int8 sdpa llama skv=%d" % skv)
    q, k, v, alpha = kvq_synth.llama_layer(skv)
    gc = kvq.QuantKVCache(1, 8, 128, skv, 64, device="cuda", bits=8)
    kvq.quantize_kv_append(gc, 0, to_dev(k), to_dev(v))
    out, *_ = run_sdpa(gc, skv, q, alpha)
    heads = [0, 5] if skv > 16384 else list(range(8))
    refs = []
    for h in heads:
        oc = _oracle_cache(np.ascontiguousarray(k[:, h:h + 1]), np.ascontiguousarray(v[:, h:h + 1]))
        refs.append(oracle.sdpa(oc, skv, np.ascontiguousarray(q[:, 8 * h:8 * h + 8]), alpha))
    got = np.concatenate([out[:, 8 * h:8 * h + 8] for h in heads], axis=1)
    check_attention(got, np.concatenate(refs, axis=1), MFMA_REL_L2, label="int8 llama")
    if skv <= 16384:  # the vector-ALU kernel on the same cache
        out_v, *_ = run_sdpa(gc, skv, q, alpha, kernel=kvq.KERNEL_VALU)
        check_attention(out_v, np.concatenate(refs, axis=1), REL_L2, label="int8 llama valu")


def test_closer_to_float_attention_than_int4():
    """The point of the wider codes: on the same rows the 8-bit cache's output
    is much nearer the unquantised attention than the int4 cache's."""
    note("int8 vs int4 error")
    q, k, v, alpha = kvq_synth.llama_layer(2048)
    outs = {}
    for bits in (4, 8):
        gc = kvq.QuantKVCache(1, 8, 128, 2048, 64, device="cuda", bits=bits)
        kvq.quantize_kv_append(gc, 0, to_dev(k), to_dev(v))
        outs[bits], *_ = run_sdpa(gc, 2048, q, alpha)
    # float64 attention on the unquantised rows, on the CPU
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    exact = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(k.astype(np.float64)), torch.from_numpy(v.astype(np.float64)), scale=alpha,
        enable_gqa=True)[:, :, 0].numpy()
    e4 = np.linalg.norm(outs[4] - exact)
    e8 = np.linalg.norm(outs[8] - exact)
    assert e8 < e4 / 8, (e4, e8)


# ------------------------------------------------------------- decode step

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("length", [0, 511, 512, 1000])
def test_decode_step(kernel, length):
    """Append + attention in one call on the 8-bit cache (the append inside
    the matrix-core kernel, or append, vector-ALU partial and reduce): cache
    bit for bit as the append alone, output bit for bit as the separate calls
    with a forced kernel (within the tolerance with AUTO), and near the
    oracle."""
    note("int8 decode step len=%d kernel=%d" % (length, kernel))
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    cap = 1024 + 8
    oc = oracle.Cache(1, 8, 128, cap, 64, bits=8)
    if length:
        oc.append(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    kn = np.ascontiguousarray(k[:, :, length:length + 1])
    vn = np.ascontiguousarray(v[:, :, length:length + 1])
    g1, g2 = gpu_cache_from_oracle(oc), gpu_cache_from_oracle(oc)
    qd, knd, vnd = to_dev(q), to_dev(kn), to_dev(vn)
    out1 = kvq.decode_step(g1, length, knd, vnd, qd, alpha, kernel=kernel)
    kvq.quantize_kv_append(g2, length, knd, vnd)
    out2 = kvq.sdpa_int4(g2, length + 1, qd, alpha, kernel=kernel)
    torch.cuda.synchronize()
    oc.append(kn, vn, length)
    assert_cache_equal(g1, oc)
    got = out1.cpu().numpy()
    if kernel in (kvq.KERNEL_AUTO, kvq.KERNEL_MFMA):  # another split of the rows
        check_attention(got, out2.cpu().numpy(), GATE[kernel], label="int8 step vs separate calls")
    else:
        assert np.array_equal(got, out2.cpu().numpy())
    check_attention(got, oracle.sdpa(oc, length + 1, q, alpha), GATE[kernel], label="int8 step")


@pytest.mark.parametrize("length", [511, 1023])
def test_decode_step_fp32_inputs(length):
    """fp32 K/V rows and fp32 q (the split-query matrix-core path)."""
    note("int8 decode step fp32 len=%d" % length)
    q, k, v, alpha = kvq_synth.tiny_decode(skv=length + 1)
    B, Hkv, _, D = k.shape
    oc = oracle.Cache(B, Hkv, D, length + 1, 64, bits=8)
    oc.append(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    kn = np.ascontiguousarray(k[:, :, length:])
    vn = np.ascontiguousarray(v[:, :, length:])
    g = gpu_cache_from_oracle(oc)
    out = kvq.decode_step(g, length, to_dev(kn), to_dev(vn), to_dev(q), alpha, kernel=kvq.KERNEL_MFMA_WAVE)
    torch.cuda.synchronize()
    oc.append(kn, vn, length)
    assert_cache_equal(g, oc)
    check_attention(out.cpu().numpy(), oracle.sdpa(oc, length + 1, q, alpha), MFMA_REL_L2, label="int8 step fp32")


@pytest.mark.parametrize("kernel", [kvq.KERNEL_MFMA_SPLIT])
def test_matrix_core_variants_refuse_int8(kernel):
    note("int8 refused by kernel=%d" % kernel)
    gc = kvq.QuantKVCache(1, 8, 128, 1024, 64, device="cuda", bits=8)
    q = torch.zeros((1, 64, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        run_sdpa(gc, 1024, q.cpu().numpy(), 0.1, kernel=kernel)
    assert e.value.status == -7

"""GPU parity of the decode step (kvq_decode_step): append the current
token's K/V row, then attention over the rows up to and including it.

The fused path (append inside the attention kernel) must leave the cache bit
for bit as kvq_quantize_kv_append does. With a forced one-wavefront kernel its
output equals the separate calls with the same kernel bit for bit; with AUTO
(the eight-wavefront workgroups, another split of the rows) it matches them
within the attention tolerance. Both are also checked against the float64
oracle."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import assert_cache_equal, check_attention, gpu_cache_from_oracle, note, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4  # the matrix-core gate of test_gpu_sdpa.py


def _setup(k, v, length, cap, G=64):
    """Oracle cache holding rows [0, length) of k, v; the new row is `length`."""
    B, Hkv, S, D = k.shape
    oc = oracle.Cache(B, Hkv, D, cap, G)
    if length:
        oc.append(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    return oc


def _new_row(k, v, length):
    return (np.ascontiguousarray(k[:, :, length:length + 1]), np.ascontiguousarray(v[:, :, length:length + 1]))


def _step_and_compare(q, k, v, alpha, length, cap, kernel=kvq.KERNEL_AUTO, G=64):
    oc = _setup(k, v, length, cap, G)
    kn, vn = _new_row(k, v, length)
    g1 = gpu_cache_from_oracle(oc)
    g2 = gpu_cache_from_oracle(oc)
    qd, knd, vnd = to_dev(q), to_dev(kn), to_dev(vn)
    out1 = kvq.decode_step(g1, length, knd, vnd, qd, alpha, kernel=kernel)
    kvq.quantize_kv_append(g2, length, knd, vnd)
    # the step picks its attention kernel by the same rule as kvq_sdpa_int4
    out2 = kvq.sdpa_int4(g2, length + 1, qd, alpha, kernel=kernel)
    torch.cuda.synchronize()
    oc.append(kn, vn, length)
    assert_cache_equal(g1, oc)
    got = out1.cpu().numpy()
    if kernel in (kvq.KERNEL_AUTO, kvq.KERNEL_MFMA):
        check_attention(got, out2.cpu().numpy(), REL_L2, label="decode step vs separate calls len=%d" % length)
    else:
        assert np.array_equal(got, out2.cpu().numpy()), "decode step differs from the separate calls"
    check_attention(got, oracle.sdpa(oc, length + 1, q, alpha), REL_L2, label="decode step len=%d" % length)


@pytest.mark.parametrize("length", [0, 1, 511, 512, 1000, 4095])
def test_decode_step_llama(length):
    note("decode step llama len=%d" % length)
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    _step_and_compare(q, k, v, alpha, length, cap=4096 + 8)


@pytest.mark.parametrize("length", [0, 511, 512, 4095])
def test_decode_step_fused_forced(length):
    """The fused path (append inside the one-wavefront kernel) at sizes where
    AUTO would not take it."""
    note("decode step fused forced len=%d" % length)
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    _step_and_compare(q, k, v, alpha, length, cap=4096 + 8, kernel=kvq.KERNEL_MFMA_WAVE)


@pytest.mark.parametrize("length", [511, 1023])
@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
def test_decode_step_fp32_inputs(length, kernel):
    note("decode step fp32 len=%d kernel=%d" % (length, kernel))
    q, k, v, alpha = kvq_synth.tiny_decode(skv=length + 1)
    _step_and_compare(q, k, v, alpha, length, cap=length + 1, kernel=kernel)


def test_decode_step_unfused_path():
    note("decode step valu")
    q, k, v, alpha = kvq_synth.llama_layer(700)
    _step_and_compare(q, k, v, alpha, 699, cap=1024, kernel=kvq.KERNEL_VALU)


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
def test_decode_step_head_dim_256(kernel):
    note("decode step gemma D=256 kernel=%d" % kernel)
    q, k, v, alpha = kvq_synth.gemma_layer(786)
    _step_and_compare(q, k, v, alpha, 785, cap=800, kernel=kernel)


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
@pytest.mark.parametrize("Hq,Hkv,D,G,length", [(64, 2, 128, 64, 0), (64, 2, 128, 64, 1500), (20, 1, 256, 128, 999),
                                               (14, 2, 128, 32, 513)])
def test_decode_step_wide_gqa(kernel, Hq, Hkv, D, G, length):
    """Query heads of one KV head in several blocks: every block quantises the
    new row into the same cache bytes and attends over it."""
    note("decode step wide gqa Hq%d Hkv%d D%d G%d len=%d kernel=%d" % (Hq, Hkv, D, G, length, kernel))
    S = length + 1
    q = kvq_synth.normal((1, Hq, D), [88, Hq, D, length, 0]).astype(np.float16)
    k = kvq_synth.normal((1, Hkv, S, D), [88, Hq, D, length, 1]).astype(np.float16)
    v = kvq_synth.normal((1, Hkv, S, D), [88, Hq, D, length, 2]).astype(np.float16)
    _step_and_compare(q, k, v, 1 / np.sqrt(D), length, cap=(S + 15) // 8 * 8, kernel=kernel, G=G)


@pytest.mark.parametrize("B,Hq,Hkv,D,G,length", [(3, 24, 3, 128, 64, 2999), (2, 16, 4, 256, 64, 1500),
                                                 (2, 64, 8, 128, 64, 700), (4, 8, 1, 128, 32, 63)])
def test_decode_step_batches(B, Hq, Hkv, D, G, length):
    """Batch entries index their own cache rows, partials and outputs in the
    eight- (four-) wavefront workgroups, at lengths from two workgroups per
    head down to one tile."""
    note("decode step batch B%d Hq%d Hkv%d D%d G%d len=%d" % (B, Hq, Hkv, D, G, length))
    S = length + 1
    q = kvq_synth.normal((B, Hq, D), [90, B, Hq, D, 0]).astype(np.float16)
    k = kvq_synth.normal((B, Hkv, S, D), [90, B, Hq, D, 1]).astype(np.float16)
    v = kvq_synth.normal((B, Hkv, S, D), [90, B, Hq, D, 2]).astype(np.float16)
    _step_and_compare(q, k, v, 1 / np.sqrt(D), length, cap=(S + 7) // 8 * 8, G=G)


def test_decode_steps_in_sequence():
    """Three tokens decoded one after another into one cache."""
    note("decode steps in sequence")
    q, k, v, alpha = kvq_synth.llama_layer(1027)
    length = 1024
    oc = _setup(k, v, length, cap=1100)
    g = gpu_cache_from_oracle(oc)
    qd = to_dev(q)
    for t in range(length, length + 3):
        kn, vn = _new_row(k, v, t)
        out = kvq.decode_step(g, t, to_dev(kn), to_dev(vn), qd, alpha)
        torch.cuda.synchronize()
        oc.append(kn, vn, t)
        check_attention(out.cpu().numpy(), oracle.sdpa(oc, t + 1, q, alpha), REL_L2, label="step %d" % t)
    assert_cache_equal(g, oc)

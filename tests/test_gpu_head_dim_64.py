"""GPU parity at head_dim 64 on the matrix-core kernels, whose 16 value
columns there are half octets of the row (four dimensions each): split-K
attention (one-wavefront kernel and AUTO), its partial states, the decode step
(fused append, eight-wavefront workgroups or one-wavefront kernel) and the
single-launch step, on int4 and int8 caches, against the float64 oracle.

Shapes: a 64-wide head with 32 query heads over 8 KV heads (the layout of
small Llama-family models), plain multi-head attention, and more query heads
per KV head than one score instruction's 16 columns hold (run in blocks)."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import assert_cache_equal, check_attention, gpu_cache_from_oracle, note, run_sdpa, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4  # the matrix-core gate of test_gpu_sdpa.py
D = 64

# (B, Hq, Hkv, G): n_rep 4, 4, 1, 32 (four blocks of 8 at one group per
# head), 12 (three blocks of 4 at two groups), 16 (four blocks of 4): a
# block holds at most 8 (head, group) score columns
SHAPES = [(1, 32, 8, 64), (2, 8, 2, 32), (1, 4, 4, 64), (1, 64, 2, 64), (1, 12, 1, 32), (2, 16, 1, 32)]


def _inputs(B, Hq, Hkv, S, seed, qdt=np.float16):
    q = kvq_synth.normal((B, Hq, D), seed + [0]).astype(qdt)
    k = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, S, D), seed + [1]))
    v = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, S, D), seed + [2]))
    return q, k, v, 1 / np.sqrt(D)


def _oracle_cache(k, v, length, cap, G, bits):
    B, Hkv, _, _ = k.shape
    oc = oracle.Cache(B, Hkv, D, cap, G, bits=bits)
    if length:
        oc.append(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    return oc


@pytest.mark.parametrize("kernel", [kvq.KERNEL_MFMA_WAVE, kvq.KERNEL_AUTO])
@pytest.mark.parametrize("B,Hq,Hkv,G", SHAPES)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("qdt", [np.float16, np.float32])
def test_sdpa(kernel, B, Hq, Hkv, G, bits, qdt):
    note("d64 sdpa B%d Hq%d Hkv%d G%d bits%d q%s kernel=%d" % (B, Hq, Hkv, G, bits, np.dtype(qdt).name, kernel))
    S = 2100
    q, k, v, alpha = _inputs(B, Hq, Hkv, S, [190, B, Hq, Hkv, G, bits], qdt)
    oc = _oracle_cache(k, v, S, S + 3, G, bits)  # (an odd capacity: the heads' rows start anywhere)
    out, *_ = run_sdpa(gpu_cache_from_oracle(oc), S, q, alpha, kernel=kernel)
    check_attention(out, oracle.sdpa(oc, S, q, alpha), REL_L2, label="d64 sdpa")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("skv,chunk", [(1, 512), (33, 512), (511, 512), (513, 512), (1000, 100), (1000, 64),
                                       (1500, 256), (1000, 1), (1000, 3)])
def test_ragged(bits, skv, chunk):
    note("d64 ragged skv=%d chunk=%d bits=%d" % (skv, chunk, bits))
    q, k, v, alpha = _inputs(1, 8, 2, 1536, [191, bits])
    oc = _oracle_cache(k, v, 1536, 1536, 64, bits)
    out, *_ = run_sdpa(gpu_cache_from_oracle(oc), skv, q, alpha, chunk=chunk, kernel=kvq.KERNEL_MFMA_WAVE)
    check_attention(out, oracle.sdpa(oc, skv, q, alpha), REL_L2, label="d64 ragged")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("G", [32, 64])
def test_partials_match_oracle(bits, G):
    """The partial state of include/kvq.h (m the chunk maximum, l >= 1, acc)
    for every (head, chunk)."""
    note("d64 partials bits=%d G=%d" % (bits, G))
    skv, chunk = 4001, 512
    q, k, v, alpha = _inputs(1, 32, 8, skv, [192, bits, G])
    oc = _oracle_cache(k, v, skv, skv + 7, G, bits)
    _, m, l, acc = run_sdpa(gpu_cache_from_oracle(oc), skv, q, alpha, chunk=chunk, kernel=kvq.KERNEL_MFMA_WAVE)
    rm, rl, racc = oracle.sdpa_partials(oc, skv, q, alpha, chunk)
    np.testing.assert_allclose(m, rm, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(l, rl, rtol=1e-4)
    assert np.all(l >= 1.0 - 1e-5)
    check_attention(acc / l[..., None], racc / rl[..., None], REL_L2, label="d64 partials acc/l")


def _step(q, k, v, alpha, length, cap, G, bits, kernel):
    oc = _oracle_cache(k, v, length, cap, G, bits)
    kn = np.ascontiguousarray(k[:, :, length:length + 1])
    vn = np.ascontiguousarray(v[:, :, length:length + 1])
    g = gpu_cache_from_oracle(oc)
    out = kvq.decode_step(g, length, to_dev(kn), to_dev(vn), to_dev(q), alpha, kernel=kernel)
    torch.cuda.synchronize()
    oc.append(kn, vn, length)
    assert_cache_equal(g, oc)
    return out.cpu().numpy(), oc


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("length", [0, 1, 511, 4095, 20000])
def test_decode_step(kernel, bits, length):
    """Append inside the attention launch: the cache bit for bit, the output
    against the oracle."""
    note("d64 decode step len=%d bits=%d kernel=%d" % (length, bits, kernel))
    q, k, v, alpha = _inputs(1, 32, 8, length + 1, [193, bits])
    got, oc = _step(q, k, v, alpha, length, (length + 16) // 8 * 8, 64, bits, kernel)
    check_attention(got, oracle.sdpa(oc, length + 1, q, alpha), REL_L2, label="d64 step len=%d" % length)


@pytest.mark.parametrize("B,Hq,Hkv,G", SHAPES)
def test_decode_step_shapes(B, Hq, Hkv, G):
    note("d64 decode step shape B%d Hq%d Hkv%d G%d" % (B, Hq, Hkv, G))
    length = 3000
    q, k, v, alpha = _inputs(B, Hq, Hkv, length + 1, [194, B, Hq, Hkv, G])
    got, oc = _step(q, k, v, alpha, length, length + 8, G, 4, kvq.KERNEL_AUTO)
    check_attention(got, oracle.sdpa(oc, length + 1, q, alpha), REL_L2, label="d64 step shape")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("length", [0, 1000, 16383])
def test_single_launch(bits, length):
    """The single-launch step: workgroup partials merged by the last
    workgroup of each (KV head, head block), counters back at zero."""
    note("d64 single launch len=%d bits=%d" % (length, bits))
    q, k, v, alpha = _inputs(1, 64, 2, length + 1, [195, bits])
    cap = (length + 16) // 8 * 8
    oc = _oracle_cache(k, v, length, cap, 64, bits)
    kn = np.ascontiguousarray(k[:, :, length:length + 1])
    vn = np.ascontiguousarray(v[:, :, length:length + 1])
    g = gpu_cache_from_oracle(oc)
    ws = kvq.decode_workspace(g, q.shape[1], length + 1)
    out = kvq.decode_step_single_launch(g, length, to_dev(kn), to_dev(vn), to_dev(q), alpha, workspace=ws)
    torch.cuda.synchronize()
    assert not ws[:4 * q.shape[1]].any().item(), "arrival counters not reset"
    oc.append(kn, vn, length)
    assert_cache_equal(g, oc)
    check_attention(out.cpu().numpy(), oracle.sdpa(oc, length + 1, q, alpha), REL_L2, label="d64 single launch")


@pytest.mark.parametrize("skv,bits", [(131072, 4), (131072, 8), (65536, 4)])
def test_full_size(skv, bits):
    """A 64-wide layer with 32 query heads over 8 KV heads at 64K and 128K
    rows: the decode step under AUTO, every head against the oracle."""
    note("d64 full size skv=%d bits=%d" % (skv, bits))
    q, k, v, alpha = _inputs(1, 32, 8, skv, [196, skv, bits])
    got, oc = _step(q, k, v, alpha, skv - 1, skv, 64, bits, kvq.KERNEL_AUTO)
    check_attention(got, oracle.sdpa(oc, skv, q, alpha), REL_L2, label="d64 full size")

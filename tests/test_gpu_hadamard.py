"""GPU parity of the Hadamard-rotated cache (the rotation of the blog on
running Gemma 4 with TurboQuant, its "TurboQuant" section): the rotated
append must write the cache the oracle writes bit for bit (fp16 rows: the
rotation sums are exact, so both sides quantise the same fp32 values), the
rotation kernel must give the oracle's rotation (bit for bit for fp16 rows),
and attention over a rotated cache with a rotated query, rotated back, must
match the oracle within the matrix-core tolerance."""

import math

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import (META_CANARY, WORD_CANARY, assert_cache_equal, canary_cache, check_attention, host_arrays,
                         note, run_sdpa, to_dev)

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4  # the matrix-core gate of test_gpu_sdpa.py


def _rot_append_and_check(k, v, length, cap, G=64, bits=4):
    B, Hkv, n, D = k.shape
    gc = canary_cache(B, Hkv, D, cap, G, bits=bits)
    kvq.quantize_kv_append_rotated(gc, length, to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    oc = oracle.Cache(B, Hkv, D, cap, G, bits=bits)
    oc.append_rotated(k, v, length)
    rows = slice(length, length + n)
    assert_cache_equal(gc, oc, rows)
    outside = np.ones(cap, dtype=bool)
    outside[rows] = False
    for i, a in enumerate(host_arrays(gc)):
        canary = WORD_CANARY.view(np.uint32) if i < 2 else META_CANARY
        assert np.all(a[:, :, outside] == canary), "rows outside the append range were written"
    return gc, oc


@pytest.mark.parametrize("B,Hkv,D,G,n,length", [(1, 8, 128, 64, 300, 5), (2, 3, 64, 32, 77, 0),
                                                 (1, 2, 256, 64, 129, 3), (1, 4, 128, 128, 64, 1),
                                                 (1, 1, 256, 128, 1, 9)])
def test_rotated_append_bit_exact(B, Hkv, D, G, n, length):
    note("rotated append B%d Hkv%d D%d G%d n%d len%d" % (B, Hkv, D, G, n, length))
    k = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, n, D), [110, B, Hkv, D, G, n, 0]))
    v = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, n, D), [110, B, Hkv, D, G, n, 1]))
    _rot_append_and_check(k, v, length, length + n + 3, G)


def test_rotated_append_special_rows():
    note("rotated append special rows")
    D = 128
    rows = [np.zeros(D), np.full(D, 3.5), np.full(D, -1e-7), np.linspace(-5000, 5000, D),
            np.where(np.arange(D) % 9 == 0, 2000.0, 6e-8), (np.arange(D) % 2) * 2.0 ** -20,
            np.eye(D)[0] * 40000.0, np.eye(D)[D - 1] * -40000.0]
    k = np.stack(rows).astype(np.float16)[None, None]
    v = np.stack(rows[::-1]).astype(np.float16)[None, None]
    _rot_append_and_check(k, v, 2, 12)


def test_rotated_decode_appends():
    note("rotated single-row appends")
    k = kvq_synth.to_f16(kvq_synth.normal((1, 8, 6, 128), [111, 0]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, 8, 6, 128), [111, 1]))
    gc = kvq.Int4KVCache(1, 8, 128, 8, 64, device=torch.device("cuda"))
    oc = oracle.Cache(1, 8, 128, 8, 64)
    for t in range(6):
        kt, vt = np.ascontiguousarray(k[:, :, t:t + 1]), np.ascontiguousarray(v[:, :, t:t + 1])
        kvq.quantize_kv_append_rotated(gc, t, to_dev(kt), to_dev(vt))
        oc.append_rotated(kt, vt, t)
    torch.cuda.synchronize()
    assert_cache_equal(gc, oc, slice(0, 6))


def test_outlier_rotated_append():
    """The outlier workload's 4096-row append (Student-t keys with boosted
    channels), rotated, at row 61440 of a 65536-row cache."""
    note("rotated outlier append 4096 at 61440")
    _, k, v, _ = kvq_synth.outlier_kv()
    kn = np.ascontiguousarray(k[:, :, 61440:])
    vn = np.ascontiguousarray(v[:, :, 61440:])
    _rot_append_and_check(kn, vn, 61440, 65536)


def test_rotated_append_rejects_fp32():
    note("rotated append fp32 rejected")
    gc = kvq.Int4KVCache(1, 1, 128, 4, 64, device=torch.device("cuda"))
    x = torch.zeros((1, 1, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.quantize_kv_append_rotated(gc, 0, x, x)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("rows", [1, 7, 1000])
def test_rotate_fp16_bit_exact(D, rows):
    note("rotate fp16 D%d rows%d" % (D, rows))
    x = kvq_synth.to_f16(kvq_synth.normal((rows, D), [112, D, rows]) * 30.0)
    got = kvq.hadamard_rotate(to_dev(x)).cpu().numpy()
    want = oracle.hadamard(x).astype(np.float32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotate_fp32_and_in_place(D):
    note("rotate fp32 D%d" % D)
    x = kvq_synth.normal((33, D), [113, D])
    want = oracle.hadamard(x)
    xd = to_dev(x)
    got = kvq.hadamard_rotate(xd).cpu().numpy()
    assert np.allclose(got, want, rtol=2e-7, atol=1e-7)
    kvq.hadamard_rotate(xd, out=xd)  # in place
    assert np.array_equal(xd.cpu().numpy(), got)
    back = kvq.hadamard_rotate(xd).cpu().numpy()  # its own inverse
    assert np.allclose(back, x, rtol=1e-6, atol=1e-6)


def _rotated_attention(q, k, v, alpha, cap=None, chunk=512, kernel=kvq.KERNEL_AUTO, label=""):
    B, Hkv, S, D = k.shape
    gc = kvq.Int4KVCache(B, Hkv, D, cap or S, 64, device=torch.device("cuda"))
    kvq.quantize_kv_append_rotated(gc, 0, to_dev(k), to_dev(v))
    qr = kvq.hadamard_rotate(to_dev(q)).cpu().numpy()
    out, _, _, _ = run_sdpa(gc, S, qr, alpha, chunk=chunk, kernel=kernel)
    got = kvq.hadamard_rotate(torch.from_numpy(out).cuda()).cpu().numpy()
    oc = oracle.Cache(B, Hkv, D, cap or S, 64)
    oc.append_rotated(k, v, 0)
    assert_cache_equal(gc, oc, slice(0, S))
    return check_attention(got, oracle.sdpa_rotated(oc, S, q, alpha), REL_L2, label=label)


@pytest.mark.parametrize("skv", [1, 700, 4096])
def test_rotated_attention_llama(skv):
    note("rotated attention llama skv=%d" % skv)
    q, k, v, alpha = kvq_synth.llama_layer(skv)
    _rotated_attention(q, k, v, alpha, label="rotated llama %d" % skv)


def test_rotated_attention_outlier():
    note("rotated attention outlier 8192")
    q, k, v, alpha = kvq_synth.outlier_kv(total=8192)
    _rotated_attention(q, k, v, alpha, label="rotated outlier")


@pytest.mark.parametrize("kernel", [kvq.KERNEL_VALU, kvq.KERNEL_MFMA_WAVE])
def test_rotated_attention_kernels(kernel):
    note("rotated attention kernel %d" % kernel)
    q, k, v, alpha = kvq_synth.llama_layer(1500)
    _rotated_attention(q, k, v, alpha, kernel=kernel, label="rotated kernel %d" % kernel)


def test_rotated_attention_gemma():
    note("rotated attention gemma D=256")
    q, k, v, alpha = kvq_synth.gemma_layer(786)
    _rotated_attention(q, k, v, alpha, label="rotated gemma")


# ------------------------------------------------------- rotated decode step

def _rot_step_case(q, k, v, alpha, length, cap, kernel, q_dev=None, out=None, bits=4):
    """Rows [0, length) rotated into the cache by the oracle; the step rotates
    and appends row `length` and attends over rows 0..length. Returns the GPU
    output and the oracle cache after the same append."""
    B, Hkv, _, D = k.shape
    oc = oracle.Cache(B, Hkv, D, cap, 64, bits=bits)
    if length:
        oc.append_rotated(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    kn = np.ascontiguousarray(k[:, :, length:length + 1])
    vn = np.ascontiguousarray(v[:, :, length:length + 1])
    from _gpu_common import gpu_cache_from_oracle
    g = gpu_cache_from_oracle(oc)
    got = kvq.decode_step_rotated(g, length, to_dev(kn), to_dev(vn), to_dev(q) if q_dev is None else q_dev, alpha,
                                  kernel=kernel, out=out)
    torch.cuda.synchronize()
    oc.append_rotated(kn, vn, length)
    assert_cache_equal(g, oc)
    return got.cpu().numpy(), oc


GATES = {kvq.KERNEL_VALU: 2e-5}


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE, kvq.KERNEL_MFMA_SPLIT, kvq.KERNEL_VALU])
@pytest.mark.parametrize("length", [0, 700, 4095])
def test_rotated_decode_step_llama(kernel, length):
    """The fused path (one-wavefront kernel: query rotated in its prologue,
    rows in its append, output in the reduce) and the fallbacks agree with
    the oracle's attention over the rotated cache, rotated back."""
    note("rotated step llama len=%d kernel=%d" % (length, kernel))
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    got, oc = _rot_step_case(q, k, v, alpha, length, 4096 + 8, kernel)
    check_attention(got, oracle.sdpa_rotated(oc, length + 1, q, alpha), GATES.get(kernel, 1e-4),
                    label="rotated step")


@pytest.mark.parametrize("B,Hkv,D,G,n,length", [(1, 8, 128, 64, 300, 5), (1, 2, 256, 64, 129, 3),
                                                 (1, 4, 128, 128, 64, 1)])
def test_rotated_append_int8_bit_exact(B, Hkv, D, G, n, length):
    """The rotated append into an 8-bit cache (bytes instead of nibbles)."""
    note("rotated append int8 B%d Hkv%d D%d G%d n%d len%d" % (B, Hkv, D, G, n, length))
    k = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, n, D), [111, B, Hkv, D, G, n, 0]))
    v = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, n, D), [111, B, Hkv, D, G, n, 1]))
    _rot_append_and_check(k, v, length, length + n + 3, G, bits=8)


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE, kvq.KERNEL_VALU])
@pytest.mark.parametrize("length", [0, 700, 4095])
def test_rotated_decode_step_int8(kernel, length):
    """The rotated step on an 8-bit cache: the fused one-wavefront path with
    byte operands and the vector-ALU fallback, against the oracle."""
    note("rotated step int8 len=%d kernel=%d" % (length, kernel))
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    got, oc = _rot_step_case(q, k, v, alpha, length, 4096 + 8, kernel, bits=8)
    check_attention(got, oracle.sdpa_rotated(oc, length + 1, q, alpha), GATES.get(kernel, 1e-4),
                    label="rotated step int8")


def test_rotated_decode_step_matches_separate_calls():
    """The fused step against the four separate calls it replaces (rotate q,
    rotated append, attention with the fp32 rotated query, reduce, rotate the
    output): the same numbers up to the reduce's summation order."""
    note("rotated step vs separate calls")
    length = 2047
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    got, oc = _rot_step_case(q, k, v, alpha, length, 2048, kvq.KERNEL_MFMA_WAVE)
    from _gpu_common import gpu_cache_from_oracle
    g = gpu_cache_from_oracle(oc)  # already holds the rotated row `length`
    qr = kvq.hadamard_rotate(to_dev(q))
    sep = kvq.sdpa_int4(g, length + 1, qr, alpha, kernel=kvq.KERNEL_MFMA_WAVE)
    kvq.hadamard_rotate(sep, out=sep)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got, sep.cpu().numpy(), rtol=1e-5, atol=1e-7)


def test_rotated_decode_step_fp32_query_in_place():
    note("rotated step fp32 q in place")
    length = 1000
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    qd = to_dev(q.astype(np.float32))
    for kernel in (kvq.KERNEL_MFMA_WAVE, kvq.KERNEL_MFMA_SPLIT):
        buf = qd.clone()
        got, oc = _rot_step_case(q, k, v, alpha, length, 1024, kernel, q_dev=buf, out=buf)
        check_attention(got, oracle.sdpa_rotated(oc, length + 1, q.astype(np.float32), alpha), 1e-4,
                        label="rotated step fp32 in place kernel=%d" % kernel)


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
def test_rotated_decode_step_gemma(kernel):
    """D = 256: the query is rotated before the attention kernel, the rows
    inside its append."""
    note("rotated step gemma kernel=%d" % kernel)
    q, k, v, alpha = kvq_synth.gemma_layer(787)
    got, oc = _rot_step_case(q, k.astype(np.float16), v.astype(np.float16), alpha, 786, 800, kernel)
    check_attention(got, oracle.sdpa_rotated(oc, 787, q, alpha), 1e-4, atol=1e-3, rtol=1e-3, label="rotated gemma")


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
@pytest.mark.parametrize("bits", [4, 8])
def test_rotated_decode_step_head_dim_64(kernel, bits):
    """D = 64: the query rotated before the attention kernel, the new rows
    inside its append (eight lanes per row), half-octet value columns."""
    note("rotated step d64 bits=%d kernel=%d" % (bits, kernel))
    length, Hq, Hkv, D = 2500, 32, 8, 64
    q = kvq_synth.normal((1, Hq, D), [90, bits, 0]).astype(np.float16)
    k = kvq_synth.to_f16(kvq_synth.normal((1, Hkv, length + 1, D), [90, bits, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, Hkv, length + 1, D), [90, bits, 2]))
    alpha = 1 / np.sqrt(D)
    got, oc = _rot_step_case(q, k, v, alpha, length, 2504, kernel, bits=bits)
    check_attention(got, oracle.sdpa_rotated(oc, length + 1, q, alpha), 1e-4, label="rotated d64")


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
@pytest.mark.parametrize("bits", [4, 8])
def test_rotated_decode_step_wide_gqa(kernel, bits):
    """32 query heads per KV head run as four blocks of eight: each block
    rotates its own queries and the new row, and all write the same bytes."""
    note("rotated step wide gqa bits=%d kernel=%d" % (bits, kernel))
    length, Hq, Hkv, D = 1500, 64, 2, 128
    q = kvq_synth.normal((1, Hq, D), [89, bits, 0]).astype(np.float16)
    k = kvq_synth.to_f16(kvq_synth.normal((1, Hkv, length + 1, D), [89, bits, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, Hkv, length + 1, D), [89, bits, 2]))
    alpha = 1 / np.sqrt(D)
    got, oc = _rot_step_case(q, k, v, alpha, length, 1512, kernel, bits=bits)
    check_attention(got, oracle.sdpa_rotated(oc, length + 1, q, alpha), 1e-4, label="rotated wide gqa")


def test_rotated_decode_step_auto_kernel_choice_64k():
    """At 64K rows of the Llama layer AUTO runs the rotated step on the
    one-wavefront kernel (the workgroups would stream 256 rows per wavefront):
    the same cache bytes and output bits as forcing that kernel, whose
    arithmetic the oracle tests above check."""
    note("rotated step auto at 64K")
    skv = 65536
    q, k, v, alpha = kvq_synth.llama_layer(skv)
    outs, caches = [], []
    for kernel in (kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE):
        g = kvq.QuantKVCache(1, 8, 128, skv, 64, device="cuda")
        kvq.quantize_kv_append_rotated(g, 0, to_dev(np.ascontiguousarray(k[:, :, :skv - 1])),
                                       to_dev(np.ascontiguousarray(v[:, :, :skv - 1])))
        out = kvq.decode_step_rotated(g, skv - 1, to_dev(np.ascontiguousarray(k[:, :, skv - 1:])),
                                      to_dev(np.ascontiguousarray(v[:, :, skv - 1:])), to_dev(q), alpha,
                                      kernel=kernel)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        caches.append(host_arrays(g))
    assert np.array_equal(outs[0], outs[1]), "AUTO's rotated step differs from the one-wavefront kernel's"
    for a, b in zip(*caches):
        assert np.array_equal(a, b)


def test_rotated_decode_step_rejects_fp32_rows():
    note("rotated step fp32 rows")
    g = kvq.QuantKVCache(1, 8, 128, 16, 64, device="cuda")
    q = torch.zeros((1, 64, 128), dtype=torch.float16, device="cuda")
    kn = torch.zeros((1, 8, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_step_rotated(g, 3, kn, kn, q, 0.1)
    assert e.value.status == -5

"""GPU parity on seeded random shapes: batch, query and KV heads, head_dim,
group size, code width, query dtype, cache capacity, context length and
chunk length drawn from one fixed seed, each case run through the decode
entry points (kvq_sdpa_int4 under AUTO and every forced kernel variant,
kvq_decode_step, kvq_decode_step_single_launch) and checked against the
float64 oracle, the appended row bit for bit. A forced variant may refuse a
shape only with KVQ_E_UNSUPPORTED, and only where its documented limits say
so. Prefill likewise over the shapes it takes (prefix, positions, heads,
head_dim, code width, query dtype, batch, spare capacity), and the rotated
decode step over the decode shapes."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import assert_cache_equal, check_attention, gpu_cache_from_oracle, note, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = {kvq.KERNEL_VALU: 2e-5}  # the vector-ALU gate; 1e-4 for the matrix-core kernels
N_CASES = 160


def _draw(i):
    """Case i: a valid shape drawn from a generator seeded by i alone."""
    rng = np.random.default_rng([20261, i])
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([g for g in (32, 64, 128) if g <= D]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    n_rep = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 32]))
    B = int(rng.choice([1, 1, 1, 2, 3]))
    bits = int(rng.choice([4, 8]))
    q32 = bool(rng.random() < 0.3)
    skv = int(rng.integers(1, 3000))
    cap = skv + int(rng.integers(1, 40))  # room for the decode step's new row
    chunk = int(rng.choice([512, 512, 256, 100, 64, 1024, 37]))
    alpha = float(rng.choice([1 / np.sqrt(D), 1.0 / 8, 1.0]))
    return dict(D=D, G=G, Hkv=Hkv, Hq=Hkv * n_rep, B=B, bits=bits, q32=q32, skv=skv, cap=cap, chunk=chunk,
                alpha=alpha)


def _inputs(c, i):
    B, Hq, Hkv, D, S = c["B"], c["Hq"], c["Hkv"], c["D"], c["skv"] + 1
    q = kvq_synth.normal((B, Hq, D), [20262, i, 0]).astype(np.float32 if c["q32"] else np.float16)
    k = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, S, D), [20262, i, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, S, D), [20262, i, 2]))
    if c["alpha"] == 1.0:  # normalised rows: scores of O(10) without overflow
        q = (q * np.float32(0.3)).astype(q.dtype)
    return q, k, v


def _gate(kernel, c):
    # softmax scale 1 takes the unscaled gate of the decode tests for every kernel
    return 1e-4 if c["alpha"] == 1.0 else REL_L2.get(kernel, 1e-4)


def _tol(c):
    return (1e-3, 1e-3) if c["alpha"] == 1.0 else (2e-3, 1e-2)


def _may_refuse(kernel, c):
    """Whether the documented limits let a forced variant refuse the shape."""
    D, G, bits, chunk = c["D"], c["G"], c["bits"], c["chunk"]
    mfma_shape = D // G <= 4
    if kernel == kvq.KERNEL_MFMA_SPLIT:
        return not mfma_shape or bits == 8 or D == 64
    if kernel == kvq.KERNEL_MFMA_WAVE:
        return not mfma_shape or chunk > 512
    if kernel == kvq.KERNEL_MFMA:
        return not mfma_shape or ((bits == 8 or D == 64) and chunk > 512)
    return False


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = _draw(i)
    note("random shape %d: %s" % (i, c))
    q, k, v = _inputs(c, i)
    skv, alpha = c["skv"], c["alpha"]
    oc = oracle.Cache(c["B"], c["Hkv"], c["D"], c["cap"], c["G"], bits=c["bits"])
    oc.append(np.ascontiguousarray(k[:, :, :skv]), np.ascontiguousarray(v[:, :, :skv]), 0)
    ref = oracle.sdpa(oc, skv, q, alpha)
    atol, rtol = _tol(c)
    qd = to_dev(q)

    # attention over the cache as it stands, every kernel variant
    for kernel in (kvq.KERNEL_AUTO, kvq.KERNEL_VALU, kvq.KERNEL_MFMA, kvq.KERNEL_MFMA_SPLIT, kvq.KERNEL_MFMA_WAVE):
        g = gpu_cache_from_oracle(oc)
        try:
            out = kvq.sdpa_int4(g, skv, qd, alpha, chunk=c["chunk"], kernel=kernel)
        except kvq.KvqError as e:
            assert e.status == -7 and _may_refuse(kernel, c), "kernel %d refused %s: %s" % (kernel, c, e)
            continue
        torch.cuda.synchronize()
        check_attention(out.cpu().numpy(), ref, _gate(kernel, c), atol=atol, rtol=rtol,
                        label="case %d kernel %d" % (i, kernel))

    # one decode step (append row skv, attend over skv + 1 rows), two ways
    kn = np.ascontiguousarray(k[:, :, skv:skv + 1])
    vn = np.ascontiguousarray(v[:, :, skv:skv + 1])
    g1, g2 = gpu_cache_from_oracle(oc), gpu_cache_from_oracle(oc)
    out1 = kvq.decode_step(g1, skv, to_dev(kn), to_dev(vn), qd, alpha, chunk=c["chunk"])
    out2 = kvq.decode_step_single_launch(g2, skv, to_dev(kn), to_dev(vn), qd, alpha)
    torch.cuda.synchronize()
    oc.append(kn, vn, skv)
    assert_cache_equal(g1, oc)
    assert_cache_equal(g2, oc)
    ref1 = oracle.sdpa(oc, skv + 1, q, alpha)
    check_attention(out1.cpu().numpy(), ref1, 1e-4, atol=atol, rtol=rtol, label="case %d decode step" % i)
    check_attention(out2.cpu().numpy(), ref1, 1e-4, atol=atol, rtol=rtol, label="case %d single launch" % i)


def test_draws_are_valid():
    """The generator yields shapes every entry point accepts (checked on the
    host side of the draw)."""
    for i in range(N_CASES):
        c = _draw(i)
        assert c["D"] % c["G"] == 0 and c["Hq"] % c["Hkv"] == 0 and c["cap"] > c["skv"]


N_PREFILL = 96


def _draw_prefill(i):
    """A prefill case the kernels take: G 64, at most 32 query heads per KV
    head (16 at D 256)."""
    rng = np.random.default_rng([20263, i])
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    n_rep = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16] + ([20, 24, 32] if D < 256 else [])))
    return dict(D=D, Hkv=Hkv, Hq=Hkv * n_rep, B=int(rng.choice([1, 1, 2])), bits=int(rng.choice([4, 8])),
                q32=bool(rng.random() < 0.3), q_start=int(rng.choice([0, int(rng.integers(1, 2500))])),
                sq=int(rng.integers(1, 80)), spare=int(rng.integers(0, 20)))


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill(i):
    c = _draw_prefill(i)
    note("random prefill %d: %s" % (i, c))
    B, Hq, Hkv, D, q_start, sq = c["B"], c["Hq"], c["Hkv"], c["D"], c["q_start"], c["sq"]
    S = q_start + sq
    q = kvq_synth.normal((B, Hq, sq, D), [20264, i, 0]).astype(np.float32 if c["q32"] else np.float16)
    k = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, S, D), [20264, i, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((B, Hkv, S, D), [20264, i, 2]))
    oc = oracle.Cache(B, Hkv, D, S + c["spare"], 64, bits=c["bits"])
    oc.append(k, v, 0)
    alpha = 1 / np.sqrt(D)
    out = kvq.sdpa_int4_prefill(gpu_cache_from_oracle(oc), q_start, to_dev(q), alpha)
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy(), oracle.sdpa_prefill(oc, q_start, q, alpha), 1e-4, label="prefill case %d" % i)


N_ROTATED = 24


@pytest.mark.parametrize("i", range(N_ROTATED))
def test_random_rotated_step(i):
    """The rotated decode step (kvq_decode_step_rotated) on random shapes: the
    rotated row bit for bit, the output against the oracle's attention over
    the rotated cache, rotated back."""
    c = _draw(1000 + i)
    note("random rotated step %d: %s" % (i, c))
    q, k, v = _inputs(c, 1000 + i)
    skv, alpha = c["skv"], c["alpha"]
    oc = oracle.Cache(c["B"], c["Hkv"], c["D"], c["cap"], c["G"], bits=c["bits"])
    oc.append_rotated(np.ascontiguousarray(k[:, :, :skv]), np.ascontiguousarray(v[:, :, :skv]), 0)
    kn = np.ascontiguousarray(k[:, :, skv:skv + 1])
    vn = np.ascontiguousarray(v[:, :, skv:skv + 1])
    g = gpu_cache_from_oracle(oc)
    out = kvq.decode_step_rotated(g, skv, to_dev(kn), to_dev(vn), to_dev(q), alpha, chunk=c["chunk"])
    torch.cuda.synchronize()
    oc.append_rotated(kn, vn, skv)
    assert_cache_equal(g, oc)
    atol, rtol = _tol(c)
    check_attention(out.cpu().numpy(), oracle.sdpa_rotated(oc, skv + 1, q, alpha), 1e-4, atol=atol, rtol=rtol,
                    label="rotated case %d" % i)

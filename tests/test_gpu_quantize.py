"""GPU parity of quantize-append: the packed cache written by the HIP kernel
must equal the oracle's bit for bit, and rows outside the appended range must
be left untouched."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import (META_CANARY, WORD_CANARY, assert_cache_equal, canary_cache, host_arrays, note, to_dev)

pytestmark = pytest.mark.gpu


def _append_and_check(k, v, length, cap, G=64, bits=4):
    """Append k, v [B][Hkv][n][D] at row `length` of a canary-filled cache of
    `cap` rows; compare the written rows with the oracle and the rest with
    the canary."""
    B, Hkv, n, D = k.shape
    gc = canary_cache(B, Hkv, D, cap, G, bits=bits)
    kvq.quantize_kv_append(gc, length, to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    oc = oracle.Cache(B, Hkv, D, cap, G, bits=bits)
    oc.append(k, v, length)
    rows = slice(length, length + n)
    assert_cache_equal(gc, oc, rows)
    got = host_arrays(gc)
    outside = np.ones(cap, dtype=bool)
    outside[rows] = False
    for i, a in enumerate(got):
        canary = WORD_CANARY.view(np.uint32) if i < 2 else META_CANARY
        assert np.all(a[:, :, outside] == canary), "rows outside the append range were written"
    return gc, oc


def test_tiny_fp32():
    note("quantize tiny fp32 1x2x1024x128")
    _, k, v, _ = kvq_synth.tiny_decode()
    _append_and_check(k, v, 0, 1024 + 32)


@pytest.mark.parametrize("B,Hkv,D,G,dt", [(2, 3, 64, 32, np.float32), (1, 2, 64, 64, np.float16),
                                          (1, 2, 128, 32, np.float16), (1, 2, 128, 128, np.float32),
                                          (2, 1, 256, 64, np.float16), (1, 3, 256, 128, np.float32)])
def test_shapes(B, Hkv, D, G, dt):
    note("quantize shape B%d Hkv%d D%d G%d %s" % (B, Hkv, D, G, np.dtype(dt).name))
    k = kvq_synth.normal((B, Hkv, 77, D), [70, D, G, 1]).astype(dt)
    v = (3 * kvq_synth.normal((B, Hkv, 77, D), [70, D, G, 2])).astype(dt)
    _append_and_check(k, v, 5, 90, G)


def _special_rows(D=128):
    rows = []
    rows.append(np.zeros(D))
    rows.append(np.full(D, -0.0))
    rows.append(np.full(D, 1.5))
    rows.append(np.full(D, -65504.0))
    rows.append(np.linspace(-65504.0, 65504.0, D))
    rows.append(np.full(D, 2.0 ** -24) * np.arange(D))          # fp16 subnormals
    rows.append(np.full(D, 0.1))                                  # not fp16-exact, constant
    rows.append(100.0 + 1e-3 * np.sin(np.arange(D)))              # narrow range, large offset
    rows.append(1e-7 * np.cos(np.arange(D)))                      # below fp16 resolution
    rows.append(np.where(np.arange(D) % 2 == 0, -0.0, 0.0))       # mixed signed zeros
    rows.append(np.where(np.arange(D) == 3, 5000.0, 0.01 * np.arange(D)))  # one outlier
    x = np.array(rows, dtype=np.float32)
    return x


@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_special_values(dt):
    note("quantize special values %s" % np.dtype(dt).name)
    x = _special_rows().astype(dt)
    k = x[None, None]
    v = -x[None, None]
    _append_and_check(k, v, 0, x.shape[0])


def _boundary_rows(D=128, G=64, L=15):
    """Groups whose quotients (x - bias) / scale sit on and right next to the
    half-integers where rint changes the code: each group holds its bias b
    and b + L s (so the scale is s) and values b + (k + 1/2 + delta) s for
    delta in {0, +-2^-22 .. +-2^-10}, in fp32; several scales, some of them
    not powers of two. L = 15 for int4 codes, 255 for int8."""
    rows = []
    deltas = [0.0] + [sgn * 2.0 ** -e for e in (22, 20, 18, 16, 14, 13, 12, 10) for sgn in (1, -1)]
    for si, s in enumerate([0.1, 0.3, 1.7, 3e-3, 7.0, 1.0, 0.0625]):
        s = float(np.float16(s))
        b = float(np.float16(-0.37 * (si + 1)))
        row = np.empty(D, dtype=np.float64)
        for g in range(D // G):
            vals = [b, b + L * s]
            k = 0
            while len(vals) < G:
                vals.append(b + ((k * 7) % L + 0.5 + deltas[k % len(deltas)]) * s)
                k += 1
            row[g * G:(g + 1) * G] = vals
        rows.append(row)
    return np.array(rows, dtype=np.float32)


def test_rounding_boundaries():
    note("quantize rounding boundaries fp32")
    x = _boundary_rows()
    _append_and_check(x[None, None], x[None, None, ::-1].copy(), 1, x.shape[0] + 2)


def test_decode_appends_one_row_at_a_time():
    note("quantize single-row appends")
    k = kvq_synth.to_f16(kvq_synth.normal((1, 8, 6, 128), [71, 1]))
    v = kvq_synth.to_f16(kvq_synth.normal((1, 8, 6, 128), [71, 2]))
    gc = canary_cache(1, 8, 128, 8)
    oc = oracle.Cache(1, 8, 128, 8)
    for t in range(6):
        kvq.quantize_kv_append(gc, t, to_dev(np.ascontiguousarray(k[:, :, t:t + 1])),
                               to_dev(np.ascontiguousarray(v[:, :, t:t + 1])))
    torch.cuda.synchronize()
    oc.append(k, v, 0)
    assert_cache_equal(gc, oc, slice(0, 6))


def test_outlier_append_into_existing_cache():
    """4096 new outlier-heavy fp16 rows appended at row 61440 of a cache whose
    first 61440 rows the oracle quantised; the whole cache must match."""
    note("quantize outlier append 4096 at 61440")
    total, prefix = 65536, 61440
    _, k, v, _ = kvq_synth.outlier_kv(total)
    oc = oracle.Cache(1, 8, 128, total)
    oc.append(k[:, :, :prefix], v[:, :, :prefix], 0)
    from _gpu_common import gpu_cache_from_oracle
    gc = gpu_cache_from_oracle(oc)
    kvq.quantize_kv_append(gc, prefix, to_dev(np.ascontiguousarray(k[:, :, prefix:])),
                           to_dev(np.ascontiguousarray(v[:, :, prefix:])))
    torch.cuda.synchronize()
    oc.append(k[:, :, prefix:], v[:, :, prefix:], prefix)
    assert_cache_equal(gc, oc)
    assert np.abs(k.astype(np.float32)).max() > 1000  # the outliers are really there


def test_llama_full_length():
    """The Llama-shaped layer at its longest context (131072 rows), fp16."""
    note("quantize llama 1x8x131072x128 fp16")
    _, k, v, _ = kvq_synth.llama_layer(131072)
    gc = canary_cache(1, 8, 128, 131072)
    kvq.quantize_kv_append(gc, 0, to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    oc = oracle.Cache(1, 8, 128, 131072)
    oc.append(k, v, 0)
    assert_cache_equal(gc, oc)

"""The Python binding checks every tensor before it calls the C ABI (which
sees only bare pointers): wrong shapes, dtypes, sizes and devices raise
ValueError before anything is enqueued. CPU only: the tensors here live in
host memory, so any call that got past the checks would be refused as a
non-CUDA tensor, never launched."""

import pytest
import torch

import quantized_kv_cache_quantize_amd as kvq

B, HKV, HQ, D, CAP = 1, 2, 8, 128, 1024


@pytest.fixture
def cache():
    return kvq.QuantKVCache(B, HKV, D, CAP, 64, device="cpu")


def _rows(n=1, dtype=torch.float16, shape=None):
    return torch.zeros(shape or (B, HKV, n, D), dtype=dtype)


def _ws(skv, chunk=512, c_extra=0):
    nc = kvq.num_chunks(skv, chunk) + c_extra
    return (torch.zeros((B, HQ, nc)), torch.zeros((B, HQ, nc)), torch.zeros((B, HQ, nc, D)))


def _raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_append_shapes(cache):
    # a 3-D row (the decode step's form) would have been read as n = 0
    _raises("shape", kvq.quantize_kv_append, cache, 0, _rows(shape=(B, HKV, D)), _rows(shape=(B, HKV, D)))
    _raises("shape", kvq.quantize_kv_append, cache, 0, _rows(shape=(B, HKV + 1, 4, D)), _rows(4))
    _raises("shape", kvq.quantize_kv_append, cache, 0, _rows(shape=(B, HKV, 4, 64)), _rows(4))
    _raises("same shape", kvq.quantize_kv_append, cache, 0, _rows(4), _rows(5))
    _raises("dtype", kvq.quantize_kv_append, cache, 0, _rows(4, torch.bfloat16), _rows(4, torch.bfloat16))
    _raises("same shape and dtype", kvq.quantize_kv_append, cache, 0, _rows(4), _rows(4, torch.float32))
    _raises("contiguous", kvq.quantize_kv_append, cache, 0, _rows(4).transpose(2, 3).contiguous().transpose(2, 3),
            _rows(4))
    # right shapes, but host memory
    _raises("CUDA", kvq.quantize_kv_append, cache, 0, _rows(4), _rows(4))
    _raises("shape", kvq.quantize_kv_append_rotated, cache, 0, _rows(shape=(B, HKV, D)), _rows(shape=(B, HKV, D)))


def test_partial_and_reduce_shapes(cache):
    q = torch.zeros((B, HQ, D), dtype=torch.float16)
    _raises("q has shape", kvq.sdpa_int4_partial, cache, 700, torch.zeros((B, 7, D), dtype=torch.float16), 0.1, 512,
            *_ws(700))
    _raises("q has shape", kvq.sdpa_int4_partial, cache, 700, torch.zeros((B + 1, HQ, D), dtype=torch.float16), 0.1,
            512, *_ws(700))
    _raises("q has shape", kvq.sdpa_int4_partial, cache, 700, torch.zeros((B, HQ, 64), dtype=torch.float16), 0.1,
            512, *_ws(700))
    # a workspace sized for a shorter context
    _raises("needs at least", kvq.sdpa_int4_partial, cache, 700, q, 0.1, 512, *_ws(300))
    _raises("needs at least", kvq.sdpa_int4, cache, 1000, q, 0.1, workspace=_ws(511))
    m, l, acc = _ws(700)
    _raises("dtype", kvq.sdpa_int4_partial, cache, 700, q, 0.1, 512, m.double(), l, acc)
    _raises("CUDA", kvq.sdpa_int4_partial, cache, 700, q, 0.1, 512, m, l, acc)
    _raises("out has shape", kvq.sdpa_int4, cache, 700, q, 0.1, out=torch.zeros((B, HQ, D + 1)), workspace=_ws(700))
    _raises("part_m has shape", kvq.sdpa_int4_reduce, m[:, :, :1], l, acc, torch.zeros((B, HQ, D)))
    _raises("out has shape", kvq.sdpa_int4_reduce, m, l, acc, torch.zeros((B, HQ, 64)))
    _raises("4-D", kvq.sdpa_int4_reduce, m, l, acc[0], torch.zeros((B, HQ, D)))


def test_decode_step_shapes(cache):
    q = torch.zeros((B, HQ, D), dtype=torch.float16)
    one = _rows(shape=(B, HKV, D))
    _raises("shape", kvq.decode_step, cache, 10, _rows(2), _rows(2), q, 0.1)
    _raises("shape", kvq.decode_step, cache, 10, _rows(shape=(B, HKV + 1, D)), one, q, 0.1)
    _raises("needs at least", kvq.decode_step, cache, 600, one, one, q, 0.1, workspace=_ws(512))
    _raises("q has shape", kvq.decode_step, cache, 10, one, one, q[:, :7].contiguous(), 0.1)
    _raises("CUDA", kvq.decode_step, cache, 10, one, one, q, 0.1)
    _raises("CUDA", kvq.decode_step, cache, 10, _rows(1), _rows(1), q, 0.1)
    _raises("shape", kvq.decode_step_rotated, cache, 10, _rows(3), _rows(3), q, 0.1)


def test_prefill_and_rotate_shapes(cache):
    _raises("4-D", kvq.sdpa_int4_prefill, cache, 0, torch.zeros((B, HQ, D), dtype=torch.float16), 0.1)
    q = torch.zeros((B, HQ, 4, D), dtype=torch.float16)
    _raises("out has shape", kvq.sdpa_int4_prefill, cache, 0, q, 0.1, out=torch.zeros((B, HQ, 5, D)))
    _raises("CUDA", kvq.sdpa_int4_prefill, cache, 0, q, 0.1)
    x = torch.zeros((4, D), dtype=torch.float16)
    _raises("out has shape", kvq.hadamard_rotate, x, out=torch.zeros((4, D + 1)))
    _raises("CUDA", kvq.hadamard_rotate, x)


def test_cache_tensors_checked():
    good = kvq.QuantKVCache(B, HKV, D, CAP, 64, device="cpu")
    t = list(good.tensors())
    bad = list(t)
    bad[2] = torch.zeros((B, HKV, CAP, 3), dtype=torch.float16)
    _raises("k_scale has shape", kvq.QuantKVCache, B, HKV, D, CAP, 64, tensors=tuple(bad))
    bad = list(t)
    bad[0] = bad[0].float()
    _raises("k_q has dtype", kvq.QuantKVCache, B, HKV, D, CAP, 64, tensors=tuple(bad))
    _raises("CUDA", kvq.QuantKVCache, B, HKV, D, CAP, 64, tensors=tuple(t))
    _raises("unsupported", kvq.QuantKVCache, B, HKV, D, CAP, 64, device="cpu", bits=5)

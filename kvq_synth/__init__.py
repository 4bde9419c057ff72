"""Seeded synthetic inputs for int4-KV decode attention.

This module only draws random numbers and arranges them into the tensors the
workloads need. It holds none of the quantisation or attention arithmetic, so
both the CPU oracle's tests and the GPU path's tests and benchmark can take
their inputs from here without sharing any of the method's code.

Every array is a pure function of its seed words: the flat array is cut into
blocks of ``BLOCK`` elements and block ``i`` is drawn from the ``i``-th child of
``numpy.random.SeedSequence(seed_words)``. The result does not depend on how
many threads draw it.

The shapes and distributions stand in for the activations the source pages
measure on (Llama 3.1 70B and Gemma 4 31B decode attention); no model weights
or datasets are involved.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

BLOCK = 1 << 22

# Workload ids used as the first seed word.
TINY, LLAMA, LLAMA_STEP, GEMMA, OUTLIER = 0, 1, 2, 3, 4
# Tensor ids used as the last seed word.
T_Q, T_K, T_V, T_GAIN_Q, T_GAIN_K, T_CHANNELS = 0, 1, 2, 3, 4, 5


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _blocked(n: int, seed_words, draw) -> np.ndarray:
    """Fill a flat float32 array of n elements block by block."""
    out = np.empty(n, dtype=np.float32)
    nblk = (n + BLOCK - 1) // BLOCK
    children = np.random.SeedSequence(list(seed_words)).spawn(max(nblk, 1))

    def work(i):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        rng = np.random.default_rng(children[i])
        out[lo:hi] = draw(rng, hi - lo)

    if nblk <= 1:
        if n:
            work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out


def normal(shape, seed_words) -> np.ndarray:
    """float32 draws from N(0, 1)."""
    n = int(np.prod(shape))
    return _blocked(n, seed_words, lambda r, m: r.standard_normal(m, dtype=np.float32)).reshape(shape)


def student_t(shape, nu: float, seed_words) -> np.ndarray:
    """float32 draws from Student's t with nu degrees of freedom."""
    n = int(np.prod(shape))
    return _blocked(n, seed_words, lambda r, m: r.standard_t(nu, m).astype(np.float32)).reshape(shape)


def uniform(shape, lo: float, hi: float, seed_words) -> np.ndarray:
    n = int(np.prod(shape))
    return _blocked(n, seed_words, lambda r, m: r.uniform(lo, hi, m).astype(np.float32)).reshape(shape)


def to_f16(x: np.ndarray) -> np.ndarray:
    """Cast a float32 draw to fp16 (round to nearest even), as the workloads
    that store fp16 activations do."""
    return x.astype(np.float16)


# ---------------------------------------------------------------- workloads

def tiny_decode(skv: int = 1024, seed: int = 0):
    """Tiny decode: batch 1, 8 query heads, 2 KV heads, head_dim 128,
    Q/K/V fp32 N(0,1). Returns (q[1,8,128], k[1,2,skv,128], v[1,2,skv,128], alpha)."""
    b, hq, hkv, d = 1, 8, 2, 128
    q = normal((b, hq, d), [TINY, skv, seed, T_Q])
    k = normal((b, hkv, skv, d), [TINY, skv, seed, T_K])
    v = normal((b, hkv, skv, d), [TINY, skv, seed, T_V])
    return q, k, v, float(np.float32(1.0 / np.sqrt(128.0)))


def llama_layer(skv: int, layer: int = 0, workload: int = LLAMA):
    """Llama-3.1-70B-shaped decode layer: batch 1, 64 query heads, 8 KV heads,
    head_dim 128; Q, K, V fp16 from N(0,1). Returns (q, k, v, alpha)."""
    b, hq, hkv, d = 1, 64, 8, 128
    q = to_f16(normal((b, hq, d), [workload, skv, layer, T_Q]))
    k = to_f16(normal((b, hkv, skv, d), [workload, skv, layer, T_K]))
    v = to_f16(normal((b, hkv, skv, d), [workload, skv, layer, T_V]))
    return q, k, v, float(np.float32(1.0 / np.sqrt(128.0)))


def _rms_gain(x: np.ndarray, gain: np.ndarray) -> np.ndarray:
    """Rows scaled to unit RMS over the last axis, then times a per-channel
    gain. This shapes the input like Gemma's normalised Q/K; it is input
    preparation, not part of the attention method."""
    x64 = x.astype(np.float64)
    rms = np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True))
    return (x64 / rms * gain.astype(np.float64)).astype(np.float32)


def gemma_layer(skv: int, seed: int = 0):
    """Gemma-style unscaled attention: batch 1, 32 query heads, 16 KV heads,
    head_dim 256, softmax scale 1.0. Q (fp32) and K (fp16) rows have unit RMS
    times a per-channel gain ~U(0.5, 2) (one gain vector for Q, one for K);
    V fp16 N(0,1). Returns (q, k, v, alpha)."""
    b, hq, hkv, d = 1, 32, 16, 256
    gq = uniform((d,), 0.5, 2.0, [GEMMA, skv, seed, T_GAIN_Q])
    gk = uniform((d,), 0.5, 2.0, [GEMMA, skv, seed, T_GAIN_K])
    q = _rms_gain(normal((b, hq, d), [GEMMA, skv, seed, T_Q]), gq)
    k = to_f16(_rms_gain(normal((b, hkv, skv, d), [GEMMA, skv, seed, T_K]), gk))
    v = to_f16(normal((b, hkv, skv, d), [GEMMA, skv, seed, T_V]))
    return q, k, v, 1.0


def outlier_kv(total: int = 65536, seed: int = 0, n_outlier_channels: int = 4, boost: float = 20.0):
    """Outlier-heavy KV in the Llama layout (64/8/128): K ~ Student-t(3) with
    n_outlier_channels random channels per KV head multiplied by `boost`
    (the same channels for every token), V and Q ~ N(0,1); all fp16.
    Values are clipped to +-60000 so they stay finite in fp16 (the clip is
    never reached in practice at these sizes). Returns (q, k, v, alpha)."""
    b, hq, hkv, d = 1, 64, 8, 128
    k = student_t((b, hkv, total, d), 3.0, [OUTLIER, total, seed, T_K])
    ch = np.empty((hkv, n_outlier_channels), dtype=np.int64)
    rng = np.random.default_rng(np.random.SeedSequence([OUTLIER, total, seed, T_CHANNELS]))
    for h in range(hkv):
        ch[h] = rng.choice(d, size=n_outlier_channels, replace=False)
        k[:, h, :, ch[h]] *= np.float32(boost)
    np.clip(k, -60000.0, 60000.0, out=k)
    k = to_f16(k)
    v = to_f16(normal((b, hkv, total, d), [OUTLIER, total, seed, T_V]))
    q = to_f16(normal((b, hq, d), [OUTLIER, total, seed, T_Q]))
    return q, k, v, float(np.float32(1.0 / np.sqrt(128.0)))

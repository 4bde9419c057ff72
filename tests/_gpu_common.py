"""Shared helpers for the GPU parity tests: move seeded inputs and oracle
caches to the device, run the HIP path through the C ABI, and compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import quantized_kv_cache_quantize_amd as kvq

# Output tolerance of the decode attention (fp32 output vs the float64
# oracle): every element must satisfy |o - o_ref| <= ATOL + RTOL * |o_ref|.
ATOL, RTOL = 2e-3, 1e-2

WORD_CANARY = np.int32(0x5A5A5A5A)
META_CANARY = np.uint16(0x7BFE)  # fp16 65472


def note(msg: str):
    """Name the case before each GPU step so a crash report says which."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int32:
        return a.view(np.uint32)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return a


def canary_cache(B, Hkv, D, cap, G=64, bits=4) -> kvq.QuantKVCache:
    c = kvq.QuantKVCache(B, Hkv, D, cap, G, device=dev(), bits=bits)
    c.k_q.fill_(int(WORD_CANARY))
    c.v_q.fill_(int(WORD_CANARY))
    for t in (c.k_scale, c.k_bias, c.v_scale, c.v_bias):
        t.view(torch.int16).fill_(int(META_CANARY))
    return c


def gpu_cache_from_oracle(oc: oracle.Cache) -> kvq.QuantKVCache:
    """Device copy of a cache the oracle quantised on the host."""
    tensors = tuple(to_dev(a) for a in (oc.k_q, oc.v_q, oc.k_scale, oc.k_bias, oc.v_scale, oc.v_bias))
    return kvq.QuantKVCache(oc.B, oc.Hkv, oc.D, oc.cap, oc.G, tensors=tensors, bits=oc.bits)


def host_arrays(c: kvq.QuantKVCache):
    return tuple(to_host_bits(t) for t in c.tensors())


def assert_cache_equal(gc: kvq.QuantKVCache, oc: oracle.Cache, rows=None):
    names = ("k_q", "v_q", "k_scale", "k_bias", "v_scale", "v_bias")
    got = host_arrays(gc)
    for n, g in zip(names, got):
        r = getattr(oc, n)
        if rows is not None:
            g, r = g[:, :, rows], r[:, :, rows]
        bad = np.argwhere(g != r)
        assert bad.size == 0, "%s differs at %d places, first %s: got %#x want %#x" % (
            n, len(bad), tuple(bad[0]), int(g[tuple(bad[0])]), int(r[tuple(bad[0])]))


def run_sdpa(gc: kvq.QuantKVCache, skv: int, q: np.ndarray, alpha: float, chunk=512, kernel=kvq.KERNEL_AUTO,
             guard=64):
    """Partial + reduce through the C ABI with NaN-filled guard zones around
    every output; returns (out, m, l, acc) as numpy and checks the guards."""
    qd = to_dev(q)
    b, hq, d = q.shape
    nc = kvq.num_chunks(skv, chunk)
    nm = b * hq * nc
    m_buf = torch.full((nm + 2 * guard,), float("nan"), device=dev())
    l_buf = torch.full((nm + 2 * guard,), float("nan"), device=dev())
    a_buf = torch.full((nm * d + 2 * guard,), float("nan"), device=dev())
    o_buf = torch.full((b * hq * d + 2 * guard,), float("nan"), device=dev())
    m = m_buf[guard:guard + nm].view(b, hq, nc)
    l = l_buf[guard:guard + nm].view(b, hq, nc)
    acc = a_buf[guard:guard + nm * d].view(b, hq, nc, d)
    out = o_buf[guard:guard + b * hq * d].view(b, hq, d)
    kvq.sdpa_int4_partial(gc, skv, qd, alpha, chunk, m, l, acc, kernel=kernel)
    kvq.sdpa_int4_reduce(m, l, acc, out)
    torch.cuda.synchronize()
    for buf, n in ((m_buf, nm), (l_buf, nm), (a_buf, nm * d), (o_buf, b * hq * d)):
        h = buf.cpu().numpy()
        assert np.all(np.isnan(h[:guard])) and np.all(np.isnan(h[guard + n:])), "guard zone overwritten"
    return out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), acc.cpu().numpy()


def check_attention(got: np.ndarray, ref: np.ndarray, rel_l2: float, atol=ATOL, rtol=RTOL, label=""):
    """Element bound |o - ref| <= atol + rtol |ref| plus a per-head relative
    L2 gate (catches a dropped chunk that the element bound would miss at
    long context, where outputs are small)."""
    assert np.all(np.isfinite(got)), label + ": non-finite output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), "%s: |err| %.3g > bound %.3g at %s" % (label, err[worst], bound[worst], worst)
    num = np.linalg.norm((got - ref).reshape(-1, got.shape[-1]), axis=1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    r = (num / np.maximum(den, 1e-30)).max()
    assert r <= rel_l2, "%s: per-head relative L2 error %.3g > %.3g" % (label, r, rel_l2)
    return float(err.max()), float(r)

"""The entry points inside HIP graphs (torch.cuda.CUDAGraph capture on the
current stream): the library enqueues kernels only (no allocation, memset or
synchronisation), so a captured decode step, rotated decode step or prefill
call replays the same kernels. Each graph is replayed several times with
eager work and synchronisations in between, and every replay must equal the
eager call bit for bit (same kernels, same inputs), also after the static
query buffer is rewritten in place between replays."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import gpu_cache_from_oracle, host_arrays, note, to_dev

pytestmark = pytest.mark.gpu

B, HKV, HQ, D, G, CAP, LEN = 1, 2, 16, 128, 64, 4096, 2900
ALPHA = 1 / np.sqrt(D)


def _inputs(seed, rotated=False):
    k = kvq_synth.normal((B, HKV, LEN, D), [95, seed, 0]).astype(np.float16)
    v = kvq_synth.normal((B, HKV, LEN, D), [95, seed, 1]).astype(np.float16)
    oc = oracle.Cache(B, HKV, D, CAP, G)
    if rotated:
        oc.append_rotated(k, v, 0)
    else:
        oc.append(k, v, 0)
    kn = kvq_synth.normal((B, HKV, D), [95, seed, 2]).astype(np.float16)
    vn = kvq_synth.normal((B, HKV, D), [95, seed, 3]).astype(np.float16)
    q = kvq_synth.normal((B, HQ, D), [95, seed, 4]).astype(np.float16)
    q2 = kvq_synth.normal((B, HQ, D), [95, seed, 5]).astype(np.float16)
    return oc, to_dev(kn), to_dev(vn), to_dev(q), to_dev(q2)


def _replay_and_check(graph, out, want, qbuf, q2, want2, caches=()):
    side = torch.randn(1 << 16, device="cuda")
    for r in range(4):
        graph.replay()
        side.mul_(1.0001)  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, want), "replay %d differs from the eager call" % r
        for got_c, want_c in caches:
            for a, b in zip(host_arrays(got_c), want_c):
                assert np.array_equal(a, b), "replay %d: cache differs" % r
    qbuf.copy_(q2)
    for r in range(2):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want2), "replay with the new query %d differs" % r


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
@pytest.mark.parametrize("rotated", [False, True])
def test_decode_step_in_a_graph(rotated, kernel):
    """AUTO takes the four-wavefront kernel at this length; the forced
    one-wavefront kernel appends (and rotates) inside the attention kernel."""
    note("graph decode step rotated=%s kernel=%d" % (rotated, kernel))
    oc, kn, vn, q, q2 = _inputs(1 + rotated, rotated)
    base_step = kvq.decode_step_rotated if rotated else kvq.decode_step

    def step(*args, **kw):
        return base_step(*args, kernel=kernel, **kw)
    ws = kvq.partials_buffers(B, HQ, D, LEN + 1)
    # eager reference on its own cache copy, for both queries (the appended
    # row is the same each time, so the cache ends the same)
    ce = gpu_cache_from_oracle(oc)
    want = step(ce, LEN, kn, vn, q, ALPHA).clone()
    want2 = step(ce, LEN, kn, vn, q2, ALPHA).clone()
    torch.cuda.synchronize()
    want_cache = host_arrays(ce)

    cg = gpu_cache_from_oracle(oc)
    qbuf = q.clone()
    out = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        step(cg, LEN, kn, vn, qbuf, ALPHA, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cg, LEN, kn, vn, qbuf, ALPHA, out=out, workspace=ws)
    torch.cuda.synchronize()
    _replay_and_check(g, out, want, qbuf, q2, want2, caches=[(cg, want_cache)])


def test_prefill_in_a_graph():
    note("graph prefill")
    sq, q_start = 40, LEN - 40
    oc, _, _, _, _ = _inputs(3)
    q = to_dev(kvq_synth.normal((B, HQ, sq, D), [96, 0]).astype(np.float16))
    q2 = to_dev(kvq_synth.normal((B, HQ, sq, D), [96, 1]).astype(np.float16))
    gc = gpu_cache_from_oracle(oc)
    want = kvq.sdpa_int4_prefill(gc, q_start, q, ALPHA).clone()
    want2 = kvq.sdpa_int4_prefill(gc, q_start, q2, ALPHA).clone()
    qbuf = q.clone()
    out = torch.empty((B, HQ, sq, D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvq.sdpa_int4_prefill(gc, q_start, qbuf, ALPHA, out=out)
    torch.cuda.synchronize()
    _replay_and_check(g, out, want, qbuf, q2, want2)

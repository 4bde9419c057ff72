"""GPU parity of the single-launch decode step (kvq_decode_step_single_launch):
append the token's K/V row, attend over the rows up to and including it, and
merge the split-K states inside the same launch (workgroup merges in LDS,
then the last workgroup of each (batch, KV head) merges the workgroups'
partials behind an arrival counter that it resets).

Checked against the float64 oracle (cache bit for bit, output within the
attention tolerance), against the two-launch step, across consecutive calls
on one workspace (the counters must come back to zero), in HIP graph
replays, and on the shapes that take the three-launch path instead."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import assert_cache_equal, check_attention, gpu_cache_from_oracle, note, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4  # the matrix-core gate of test_gpu_sdpa.py
REL_L2_UNSCALED = 1e-4  # softmax scale 1 (test_gpu_sdpa.py)


def _setup(k, v, length, cap, G=64, bits=4):
    B, Hkv, S, D = k.shape
    oc = oracle.Cache(B, Hkv, D, cap, G, bits=bits)
    if length:
        oc.append(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    return oc


def _new_row(k, v, length):
    return (np.ascontiguousarray(k[:, :, length:length + 1]), np.ascontiguousarray(v[:, :, length:length + 1]))


def _counters_zero(ws, gc, hq):
    """The arrival counters of the workspace (the first 4 * B * Hq bytes)
    are back at zero."""
    return not ws[:4 * gc.batch * hq].any().item()


def _step(q, k, v, alpha, length, cap, G=64, bits=4, rel_l2=REL_L2, atol=2e-3, rtol=1e-2, compare_two=True):
    oc = _setup(k, v, length, cap, G, bits)
    kn, vn = _new_row(k, v, length)
    g = gpu_cache_from_oracle(oc)
    qd, knd, vnd = to_dev(q), to_dev(kn), to_dev(vn)
    ws = kvq.decode_workspace(g, q.shape[1], length + 1)
    out = kvq.decode_step_single_launch(g, length, knd, vnd, qd, alpha, workspace=ws)
    torch.cuda.synchronize()
    assert _counters_zero(ws, g, q.shape[1]), "arrival counters not reset"
    oc.append(kn, vn, length)
    assert_cache_equal(g, oc)
    got = out.cpu().numpy()
    ref = oracle.sdpa(oc, length + 1, q, alpha)
    err, rel = check_attention(got, ref, rel_l2, atol=atol, rtol=rtol, label="single-launch len=%d" % length)
    if compare_two:
        # the two-launch step on a copy of the cache before the append
        g2 = gpu_cache_from_oracle(_setup(k, v, length, cap, G, bits))
        out2 = kvq.decode_step(g2, length, knd, vnd, qd, alpha).cpu().numpy()
        check_attention(got, out2, rel_l2, atol=atol, rtol=rtol, label="single vs two launches len=%d" % length)
    return err, rel


@pytest.mark.parametrize("length", [0, 1, 127, 511, 512, 1000, 2047, 4095, 4096, 16383])
def test_llama(length):
    note("single-launch llama len=%d" % length)
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    _step(q, k, v, alpha, length, cap=(length + 16) // 8 * 8)


@pytest.mark.parametrize("skv,bits", [(65536, 4), (131072, 4), (65536, 8), (131072, 8)])
def test_llama_full_size(skv, bits):
    """The benchmark's workload: every query head, the cache bit for bit."""
    note("single-launch llama full size skv=%d bits=%d" % (skv, bits))
    q, k, v, alpha = kvq_synth.llama_layer(skv)
    err, rel = _step(q, k, v, alpha, skv - 1, cap=skv, bits=bits, compare_two=False)
    print("single-launch skv=%d bits=%d: max abs err %.3g, worst per-head rel L2 %.3g" % (skv, bits, err, rel))


@pytest.mark.parametrize("length", [32, 785, 8191])
def test_gemma_head_dim_256(length):
    note("single-launch gemma len=%d" % length)
    q, k, v, alpha = kvq_synth.gemma_layer(length + 1)
    _step(q, k, v, alpha, length, cap=length + 1, rel_l2=REL_L2_UNSCALED, atol=1e-3, rtol=1e-3)


@pytest.mark.parametrize("bits", [4, 8])
def test_fp32_inputs(bits):
    note("single-launch fp32 q/k/v bits=%d" % bits)
    q, k, v, alpha = kvq_synth.tiny_decode(skv=3000)
    _step(q, k, v, alpha, 2999, cap=3000, bits=bits)


@pytest.mark.parametrize("B,Hq,Hkv,D,G", [(2, 8, 2, 128, 64), (1, 16, 1, 128, 128), (1, 12, 4, 128, 32),
                                          (1, 8, 8, 128, 64), (2, 16, 4, 256, 64), (1, 4, 1, 256, 32),
                                          # several query-head blocks per KV head, one arrival counter each
                                          (1, 64, 2, 128, 64), (2, 32, 1, 128, 128), (1, 20, 1, 256, 128),
                                          (1, 14, 2, 128, 32)])
def test_shapes(B, Hq, Hkv, D, G):
    note("single-launch shape B%d Hq%d Hkv%d D%d G%d" % (B, Hq, Hkv, D, G))
    S = 5000
    q = kvq_synth.normal((B, Hq, D), [83, Hq, D, G, 0]).astype(np.float16)
    k = kvq_synth.normal((B, Hkv, S, D), [83, Hq, D, G, 1]).astype(np.float16)
    v = kvq_synth.normal((B, Hkv, S, D), [83, Hq, D, G, 2]).astype(np.float16)
    _step(q, k, v, 1 / np.sqrt(D), S - 1, cap=S + 8, G=G)


@pytest.mark.parametrize("D,G,Hq,Hkv", [(64, 64, 8, 2), (256, 32, 8, 2)])
def test_three_launch_shapes(D, G, Hq, Hkv):
    """Shapes outside the matrix-core kernel (D 64; eight scale groups per
    row) take append + partial + reduce inside the same workspace."""
    note("single-launch fallback D%d G%d Hq%d Hkv%d" % (D, G, Hq, Hkv))
    S = 1500
    q = kvq_synth.normal((1, Hq, D), [84, D, Hq, 0]).astype(np.float16)
    k = kvq_synth.normal((1, Hkv, S, D), [84, D, Hq, 1]).astype(np.float16)
    v = kvq_synth.normal((1, Hkv, S, D), [84, D, Hq, 2]).astype(np.float16)
    _step(q, k, v, 1 / np.sqrt(D), S - 1, cap=S, G=G, rel_l2=2e-5)


def test_steps_in_sequence_one_workspace():
    """Consecutive tokens on one cache and one workspace: each call must find
    the counters at zero and leave them so, across lengths whose workgroup
    counts differ."""
    note("single-launch steps in sequence")
    total = 9000
    q, k, v, alpha = kvq_synth.llama_layer(total)
    start = 2040
    oc = _setup(k, v, start, cap=total)
    g = gpu_cache_from_oracle(oc)
    qd = to_dev(q)
    ws = kvq.decode_workspace(g, q.shape[1], total)
    for t in list(range(start, start + 12)) + [4095, 4096, 8191, 8999]:
        if t > start + 11:
            oc = _setup(k, v, t, cap=total)
            g = gpu_cache_from_oracle(oc)
        kn, vn = _new_row(k, v, t)
        out = kvq.decode_step_single_launch(g, t, to_dev(kn), to_dev(vn), qd, alpha, workspace=ws)
        torch.cuda.synchronize()
        assert _counters_zero(ws, g, q.shape[1]), "counters not reset after step %d" % t
        oc.append(kn, vn, t)
        check_attention(out.cpu().numpy(), oracle.sdpa(oc, t + 1, q, alpha), REL_L2, label="step %d" % t)
    assert_cache_equal(g, oc)


def test_deterministic():
    note("single-launch determinism")
    q, k, v, alpha = kvq_synth.llama_layer(20000)
    oc = _setup(k, v, 19999, cap=20000)
    kn, vn = _new_row(k, v, 19999)
    outs = []
    for _ in range(3):
        g = gpu_cache_from_oracle(oc)
        out = kvq.decode_step_single_launch(g, 19999, to_dev(kn), to_dev(vn), to_dev(q), alpha)
        outs.append(out.cpu().numpy())
    assert all(np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)) for o in outs)


def test_graph_replays():
    """A captured step replayed several times, with eager work and
    synchronisations between replays: every replay equals the eager call bit
    for bit (the kernel resets its own counters, no memset is recorded)."""
    note("single-launch graph replays")
    length = 30000
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    oc = _setup(k, v, length, cap=length + 8)
    kn, vn = _new_row(k, v, length)
    g = gpu_cache_from_oracle(oc)
    qd, knd, vnd = to_dev(q), to_dev(kn), to_dev(vn)
    ws = kvq.decode_workspace(g, q.shape[1], length + 1)
    out = torch.empty((1, q.shape[1], q.shape[2]), dtype=torch.float32, device="cuda")
    eager = kvq.decode_step_single_launch(g, length, knd, vnd, qd, alpha, workspace=ws).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvq.decode_step_single_launch(g, length, knd, vnd, qd, alpha, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kvq.decode_step_single_launch(g, length, knd, vnd, qd, alpha, workspace=ws, out=out)
    for i in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager call" % i
        assert _counters_zero(ws, g, q.shape[1])
        # eager work between replays
        kvq.decode_step_single_launch(g, length, knd, vnd, qd, alpha, workspace=ws)
        torch.cuda.synchronize()
    oc.append(kn, vn, length)
    assert_cache_equal(g, oc)
    check_attention(eager.cpu().numpy(), oracle.sdpa(oc, length + 1, q, alpha), REL_L2, label="graph eager")


def test_timed_events():
    note("single-launch timed")
    length = 10000
    q, k, v, alpha = kvq_synth.llama_layer(length + 1)
    oc = _setup(k, v, length, cap=length + 8)
    kn, vn = _new_row(k, v, length)
    g1, g2 = gpu_cache_from_oracle(oc), gpu_cache_from_oracle(oc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a = kvq.decode_step_single_launch(g1, length, to_dev(kn), to_dev(vn), to_dev(q), alpha)
    b = kvq.decode_step_single_launch(g2, length, to_dev(kn), to_dev(vn), to_dev(q), alpha, events=(e0, e1))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 100.0, ms

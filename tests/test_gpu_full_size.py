"""Full-size parity of the decode step the benchmark times.

The Llama-70B-shaped layer (64 query heads on 8 KV heads, head_dim 128, fp16
N(0,1) rows) at 65536 and 131072 rows, in the launch configuration of
bench.py (kvq_decode_step, 512-row chunks, automatic kernel choice, which at
these sizes is the fused one-wavefront path): every query head's output
against the float64 oracle, the appended row bit for bit, and the rest of the
cache untouched. The 8-bit cache at 131072 rows likewise."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import check_attention, gpu_cache_from_oracle, host_arrays, note, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4  # the matrix-core gate of test_gpu_sdpa.py


@pytest.mark.parametrize("skv,bits", [(65536, 4), (131072, 4), (131072, 8)])
def test_decode_step_full_size_all_heads(skv, bits):
    note("full-size decode step skv=%d bits=%d" % (skv, bits))
    q, k, v, alpha = kvq_synth.llama_layer(skv)
    length = skv - 1
    oc = oracle.Cache(1, 8, 128, skv, 64, bits=bits)
    oc.append(np.ascontiguousarray(k[:, :, :length]), np.ascontiguousarray(v[:, :, :length]), 0)
    g = gpu_cache_from_oracle(oc)
    kn = np.ascontiguousarray(k[:, :, length:length + 1])
    vn = np.ascontiguousarray(v[:, :, length:length + 1])
    out = kvq.decode_step(g, length, to_dev(kn), to_dev(vn), to_dev(q), alpha)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    oc.append(kn, vn, length)
    names = ("k_q", "v_q", "k_scale", "k_bias", "v_scale", "v_bias")
    for n, gb in zip(names, host_arrays(g)):
        assert np.array_equal(gb, getattr(oc, n)), "%s differs from the oracle's cache" % n
    ref = oracle.sdpa(oc, skv, q, alpha)
    err, rel = check_attention(got, ref, REL_L2, label="full size skv=%d bits=%d" % (skv, bits))
    print("full size skv=%d bits=%d: max abs err %.3g, worst per-head rel L2 %.3g" % (skv, bits, err, rel))

"""GPU parity of the full-depth decode step: one decode step on each of 80
distinct layers' caches in order on one stream (the layer loop of the
README's decode-step listing, at a context the oracle checks in seconds).
Every layer's output and appended row are compared with the oracle, so a
step that read another layer's cache, workspace or row would fail."""

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import assert_cache_equal, check_attention, gpu_cache_from_oracle, note, to_dev

pytestmark = pytest.mark.gpu

LAYERS, SKV = 80, 1536


@pytest.mark.parametrize("kernel", [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_WAVE])
def test_eighty_layer_decode_step(kernel):
    """AUTO: append, four-wavefront partial and reduce per layer (a short
    context); MFMA_WAVE: the append inside the one-wavefront kernel."""
    note("layer loop %d x Skv %d kernel=%d" % (LAYERS, SKV, kernel))
    stream = torch.cuda.current_stream()
    layers = []
    for i in range(LAYERS):
        q, k, v, alpha = kvq_synth.llama_layer(SKV + 1, layer=i)
        oc = oracle.Cache(1, 8, 128, SKV + 8, 64)
        oc.append(np.ascontiguousarray(k[:, :, :SKV]), np.ascontiguousarray(v[:, :, :SKV]), 0)
        kn = np.ascontiguousarray(k[:, :, SKV:])
        vn = np.ascontiguousarray(v[:, :, SKV:])
        layers.append(dict(oc=oc, gc=gpu_cache_from_oracle(oc), q=q, qd=to_dev(q), kn=kn, vn=vn, knd=to_dev(kn),
                           vnd=to_dev(vn), alpha=alpha))
    torch.cuda.synchronize()
    outs = [kvq.decode_step(L["gc"], SKV, L["knd"], L["vnd"], L["qd"], L["alpha"], kernel=kernel, stream=stream)
            for L in layers]
    torch.cuda.synchronize()
    for i, (L, out) in enumerate(zip(layers, outs)):
        L["oc"].append(L["kn"], L["vn"], SKV)
        assert_cache_equal(L["gc"], L["oc"], slice(SKV - 1, SKV + 1))
        check_attention(out.cpu().numpy(), oracle.sdpa(L["oc"], SKV + 1, L["q"], L["alpha"]), 1e-4,
                        label="layer %d" % i)

"""The HBM read helper (a measurement aid, not a step of the method) reads
every word it is given: with all-zero data each thread's XOR is 0, so key 0
makes some thread store it, and key 1 leaves the sink alone. Sizes from one
16-byte word to a ragged multi-round buffer."""

import pytest
import torch

import quantized_kv_cache_quantize_amd as kvq
from _gpu_common import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * (2048 * 256 * 4 + 777), 64 << 20])
def test_reads_and_stores_only_on_key(nbytes):
    note("hbm_read %d bytes" % nbytes)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    kvq.hbm_read(buf, sink[:1], key=1)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]
    kvq.hbm_read(buf, sink[:1], key=0)
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 7, 7, 7]


def test_one_nonzero_word_changes_one_thread():
    """A single word of 1 at the end of a ragged buffer: the thread that reads
    it has XOR 1 (every other thread 0), so key 1 stores exactly 1."""
    note("hbm_read one word")
    n = 4 * (2048 * 256 * 3 + 5)
    buf = torch.zeros(n, dtype=torch.int32, device="cuda")
    buf[-1] = 1
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    kvq.hbm_read(buf, sink, key=1)
    torch.cuda.synchronize()
    assert int(sink.item()) == 1

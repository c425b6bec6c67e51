"""The streaming-read probe reads every word of its buffer exactly once: the
XOR of its per-workgroup results equals the XOR of the buffer's 32-bit words
(numpy on the host copy), for every access mode (contiguous, grid stride,
scattered 4 KiB blocks), workgroup counts that do
and do not divide the buffer, and a buffer that is not a whole number of a
workgroup's 32 KiB steps."""
import numpy as np
import pytest
import torch

from paged_kv_cache_405_amd import binding as B
from tests.pa_harness import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [(64 << 20) // 4, (64 << 20) // 4 + 4 * 37])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("wgs", [1, 7, 1024, 4096])
def test_probe_reads_every_word_once(words, mode, wgs):
    if mode == 2 and words % 1024:
        pytest.skip("the scattered mode reads whole 4 KiB blocks, a power of two of them")
    rng = np.random.default_rng(words % 1000 + 7 * mode + wgs)
    host = rng.integers(0, 2 ** 32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((wgs,), -1, dtype=torch.int32, device="cuda")
    B.pa_probe_stream_read(buf, sink, wgs, mode)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host)
    log(f"[gpu] probe mode {mode} wgs {wgs} words {words}: {got:#010x} vs {want:#010x}")
    assert got == want

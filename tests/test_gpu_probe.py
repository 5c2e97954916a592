"""The streaming-read probe (pa_stream_read) reads every byte it is given:
the XOR of its per-workgroup results equals the XOR of the buffer's 32-bit
words computed on the host, for sizes from one 16-byte word to a ragged
multi-megabyte buffer, for sink sizes that change the grid, and for both
read patterns (grid stride, a contiguous slab per workgroup)."""

import numpy as np
import pytest
import torch

import decode_attention_pa_amd as pa
from tests._gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("nbytes", [16, 4096, 4112, (1 << 20) + 48, 37 * (1 << 20) + 16 * 999])
@pytest.mark.parametrize("sink_len", [1, 7, 2048])
@pytest.mark.parametrize("slab", [False, True])
def test_stream_read_reads_every_word(nbytes, sink_len, slab):
    g = torch.Generator(device="cpu").manual_seed(nbytes % 1000003 + sink_len)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = host.cuda()
    sink = torch.zeros(sink_len, dtype=torch.int32, device="cuda")
    n = pa.stream_read(src, sink, slab=slab)
    torch.cuda.synchronize()
    assert n == min(sink_len, -(-nbytes // 4096))
    got = np.bitwise_xor.reduce(sink[:n].cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want, (nbytes, sink_len, slab)
    assert not sink[n:].any()              # entries past the grid untouched
    say(f"[probe] {nbytes} bytes, {n} workgroups: XOR matches")

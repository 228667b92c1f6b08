"""The streaming-read probe (measurement utility of the library) reads every
16-byte unit of its buffer exactly once: the XOR of its per-thread sinks
equals the XOR of the buffer's words, computed on the host, for buffer sizes
that do and do not divide evenly over the waves."""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("words,wgs", [(4 * 1000003, 7), (1 << 22, 64), (4, 3), (4 * 12345, 512)])
def test_read_probe_reads_every_word_once(words, wgs):
    rng = np.random.default_rng(words + wgs)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda:0")
    hda.hda_read_probe(buf, wgs, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)

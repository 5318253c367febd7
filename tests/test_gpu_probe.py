"""mqa_hbm_read_probe: the streaming read the bench measures HBM with.  Its
result has a plain definition -- the XOR of all 32-bit words of the buffer --
which numpy computes on the host."""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20, 64 << 20])
def test_probe_xor_of_buffer(nbytes):
    log(f"probe {nbytes} bytes")
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((mk.PROBE_SINK_WORDS + 7,), -1, dtype=torch.int32, device="cuda")
    mk.hbm_read_probe(src, sink)
    torch.cuda.synchronize()
    words = sink.cpu().numpy().view(np.uint32)
    assert int(np.bitwise_xor.reduce(words[:mk.PROBE_SINK_WORDS])) == int(np.bitwise_xor.reduce(host))
    assert np.all(words[mk.PROBE_SINK_WORDS:] == 0xFFFFFFFF)   # nothing written past the sink

"""GPU check of the streaming-read probe (a measurement aid): the sink must
hold the XOR of every 32-bit word of the buffer, bit for bit, for a buffer
smaller than one pass of the grid and for one that needs several."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [65536 * 3, 64 << 20])
def test_read_probe_checksum(nbytes):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from mixed_precision_attention_amd import engine as E
    host = np.random.default_rng(1234 + nbytes).integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    E.read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view("<u4"))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    E.read_probe(buf, sink)  # a second pass cancels the first
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0

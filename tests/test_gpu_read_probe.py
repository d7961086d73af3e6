"""The streaming-read probe (moe_hbm_read_probe): it reads what it says it
reads (the sink words are the XOR of each lane's 16-byte loads, checked
against numpy on a small buffer), and it refuses bad arguments before any
launch."""
import numpy as np
import pytest
import torch

import quantized_routed_expert_moe_amd as Q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("waves,depth,spans", [(8, 1, 3), (8, 2, 4), (16, 4, 8), (64, 16, 16)])
def test_read_probe_folds_every_load(waves, depth, spans):
    rng = np.random.default_rng(waves * 100 + depth)
    nbytes = waves * 1024 * spans + 512  # a ragged tail the probe must leave unread
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).copy()).cuda()
    sink = torch.full((waves * 64,), -1, dtype=torch.int32, device="cuda")
    n = Q.moe_hbm_read_probe(buf, waves, depth, sink)
    torch.cuda.synchronize()
    lpw = spans // depth * depth
    assert n == waves * lpw * 1024
    words = host[: n // 4].reshape(waves, lpw, 64, 4)
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=3), axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32).reshape(waves, 64), want)


def test_read_probe_refusals():
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256 * 64, dtype=torch.int32, device="cuda")
    with pytest.raises(Q.QmoeError, match="multiple of 8"):
        Q.moe_hbm_read_probe(buf, 12, 1, sink)
    with pytest.raises(Q.QmoeError, match="depth"):
        Q.moe_hbm_read_probe(buf, 8, 3, sink)
    with pytest.raises(Q.QmoeError, match="less than"):
        Q.moe_hbm_read_probe(buf, 128, 16, sink)
    with pytest.raises(ValueError, match="sink"):
        Q.moe_hbm_read_probe(buf, 64, 1, sink[:10])

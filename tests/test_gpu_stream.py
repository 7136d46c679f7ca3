"""The HBM measurement helpers (moe_hbm_read, moe_hbm_copy) that give the
benchmark its practical streaming ceiling: the read touches every word (the
XOR of the blocks' sink words equals the XOR of the buffer's words, computed on
the host), the copy is exact, and bad sizes are rejected."""
import numpy as np
import pytest
import torch

import moe_ffn_int4_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 3 * (1 << 20) + 16 * 7, 96 << 20])
def test_read_touches_every_word(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-(1 << 31), 1 << 31, (nbytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = host.to(DEV)
    sink = torch.zeros(moe.hbm_read_sink_words(), dtype=torch.int32, device=DEV)
    moe.hbm_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 96 << 20])
def test_copy_is_exact(nbytes):
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    moe.hbm_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_bad_sizes_rejected():
    buf = torch.zeros(64, dtype=torch.int32, device=DEV)
    sink = torch.zeros(moe.hbm_read_sink_words(), dtype=torch.int32, device=DEV)
    L = moe.lib()
    stream = moe._stream(buf.device)
    assert L.moe_hbm_read(buf.data_ptr(), 24, sink.data_ptr(), stream) == 1
    assert L.moe_hbm_read(buf.data_ptr(), 0, sink.data_ptr(), stream) == 1
    assert L.moe_hbm_copy(buf.data_ptr() + 4, buf.data_ptr(), 64, stream) == 1

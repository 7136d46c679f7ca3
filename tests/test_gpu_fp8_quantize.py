"""fp8 row quantizers on the GPU vs the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import moe_ffn_int4_amd as moe
from gpu_util import say
from oracle.fp8 import quantize_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("rows,K", [(16, 128), (48, 640), (160, 5120), (32, 8192)])
def test_weights_tiled(rows, K):
    say(f"fp8 weights: rows={rows} K={K}")
    rng = np.random.default_rng(rows * 3 + K)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[1] = 0.0
    w[2] *= np.float32(1e-9)
    w[3, 5] = 3.0  # one large weight
    q, s = moe.quantize_fp8(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    codes = moe.untile_fp8(q.cpu(), rows, K).numpy()
    c_ref, s_ref = quantize_rows(w)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(codes, c_ref)
    # the documented byte address of a few elements in the tiled buffer
    qb = q.cpu().numpy().reshape(-1)
    for r, k in [(0, 0), (rows - 1, K - 1), (5, 37 % K), (rows // 2, K // 2 + 9)]:
        t = (r // 16) * (K // 128) + k // 128
        assert qb[t * 2048 + ((k % 128) // 32) * 512 + (r % 16) * 32 + k % 32] == c_ref[r, k]


# The launch takes 1024-thread rows below 512 rows and 256-thread rows from
# 512 on; either holds a row of up to 8192 values in registers and reads a
# longer one twice. These shapes reach all four forms and both sides of 512.
@pytest.mark.parametrize("rows,K", [(37, 5120), (37, 8320), (511, 1024), (512, 1024),
                                    (600, 5120), (600, 8320)])
@pytest.mark.parametrize("ub", [1200.0, 2.5, 0.0])
def test_activations_rows(ub, rows, K):
    say(f"fp8 activations: ub={ub} rows={rows} K={K}")
    rng = np.random.default_rng(7 + rows + K)
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32) * 1.5).to(torch.bfloat16)
    x[4] = 0.0
    x[6, 100] = 40.0  # above a small bound: saturates there
    q, s = moe.quantize_fp8_rows(x.to(DEV), ub)
    torch.cuda.synchronize()
    c_ref, s_ref = quantize_rows(x.float().numpy(), ub if ub > 0 else None)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(q.cpu().numpy(), c_ref)


def test_rejects_ragged_rows():
    with pytest.raises(moe.MoEError):
        moe.quantize_fp8(torch.zeros(20, 128, device=DEV))

"""K1 quantizer on the GPU vs the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from gpu_util import say
from oracle import int4_group_quantize
from oracle import native
from test_oracle_quantize import _golden_groups, _near_tie_groups

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_quant(w: np.ndarray):
    q, s = moe.quantize_int4(torch.from_numpy(np.ascontiguousarray(w)).to(DEV))
    torch.cuda.synchronize()
    return moe.unpack_int4(q.cpu()).numpy(), s.cpu().numpy()


def _assert_same(w, codes, scales):
    c_ref, s_ref = int4_group_quantize(w)
    np.testing.assert_array_equal(codes, c_ref)
    np.testing.assert_array_equal(scales.view(np.uint32), s_ref.view(np.uint32))


def test_hand_worked_groups():
    say("quantize: hand-worked groups")
    groups = _golden_groups()
    w = np.stack([g[1] for g in groups])
    codes, scales = _gpu_quant(w)
    for i, (name, _, scale_bits, want) in enumerate(groups):
        assert scales.view(np.uint32)[i, 0] == scale_bits, name
        np.testing.assert_array_equal(codes[i], want, err_msg=name)


def test_near_ties():
    say("quantize: near ties")
    w = _near_tie_groups(np.random.default_rng(11))
    _assert_same(w, *_gpu_quant(w))


@pytest.mark.parametrize("rows,K", [(1, 128), (3, 384), (257, 1024), (1000, 5120), (77, 8192)])
def test_random_shapes(rows, K):
    say(f"quantize: rows={rows} K={K}")
    rng = np.random.default_rng(rows * 7 + K)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[:: 5] *= np.float32(2e-5)  # some groups under the 1e-6 clamp
    if rows > 2:
        w[1, :128] = 0.0
    _assert_same(w, *_gpu_quant(w))


def test_zero_rows_is_a_no_op():
    q = torch.full((0, 64), 7, dtype=torch.uint8, device=DEV)
    s = torch.empty(0, 1, dtype=torch.float32, device=DEV)
    moe.quantize_int4(torch.empty(0, 128, device=DEV), q, s)
    torch.cuda.synchronize()


def test_rejects_bad_group_multiple():
    with pytest.raises(moe.MoEError):
        moe.quantize_int4(torch.zeros(4, 100, device=DEV))


def test_full_size_expert_matrix():
    """One 8192 x 5120 expert matrix drawn on the GPU, checked against the C oracle."""
    say("quantize: full-size W1 of a 5120 x 8192 expert")
    cfg = W.config(3)
    w = W.gen_expert_weight(cfg, "w1", 5, DEV)
    q, s = moe.quantize_int4(w)
    torch.cuda.synchronize()
    c_ref, s_ref = native.quantize_int4(w.cpu().numpy())
    np.testing.assert_array_equal(moe.unpack_int4(q.cpu()).numpy(), c_ref)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("rows,K", [(16, 128), (48, 384), (160, 5120)])
def test_tiled_layout_holds_the_same_codes(rows, K):
    """moe_quantize_int4_tiled: same codes and scales, 16-row tile order."""
    say(f"quantize tiled: rows={rows} K={K}")
    rng = np.random.default_rng(rows + K)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[3::7] *= np.float32(1e-5)
    q, s = moe.quantize_int4(torch.from_numpy(w).to(DEV), tiled=True)
    torch.cuda.synchronize()
    codes = moe.unpack_int4(moe.untile_int4(q.cpu(), rows, K)).numpy()
    scales = moe.untile_scales(s.cpu(), rows, K).numpy()
    _assert_same(w, codes, scales)
    # spot-check the documented address formula on raw bytes
    qb, sb = q.cpu().numpy().reshape(-1), s.cpu().numpy().reshape(-1)
    c_ref, s_ref = int4_group_quantize(w)
    for (r, k) in [(0, 0), (rows - 1, K - 1), (17 % rows, 130 % K), (rows // 2, K // 2 + 3)]:
        t = (r // 16) * (K // 128) + k // 128
        byte = int(qb[t * 1024 + ((k % 128) // 32) * 256 + (r % 16) * 16 + (k % 32) // 2])
        nib = (byte >> 4) if k % 2 else (byte & 15)
        assert (nib - 16 if nib >= 8 else nib) == c_ref[r, k]
        assert sb[t * 16 + r % 16] == s_ref[r, k // 128]


def test_tiled_rejects_ragged_rows():
    with pytest.raises(moe.MoEError):
        moe.quantize_int4(torch.zeros(20, 128, device=DEV), tiled=True)


@pytest.mark.parametrize("rows,K", [(16, 128), (48, 384), (8192, 5120)])
def test_pack_bf16_tiled(rows, K):
    say(f"pack bf16: rows={rows} K={K}")
    src = torch.randn(rows, K, device=DEV).to(torch.bfloat16)
    dst = moe.pack_bf16_tiled(src)
    torch.cuda.synchronize()
    assert torch.equal(moe.untile_bf16(dst, rows, K), src)
    flat, ref = dst.reshape(-1).cpu(), src.cpu()
    for (r, k) in [(0, 0), (rows - 1, K - 1), (5, 37 % K), (rows // 2, K // 2 + 9)]:
        t = (r // 16) * (K // 128) + k // 128
        at = t * 2048 + ((k % 128) // 32) * 512 + (r % 16) * 32 + (k % 32)
        assert flat[at] == ref[r, k]


@pytest.mark.parametrize("group", [128, 64, 32])
@pytest.mark.parametrize("rows,K", [(16, 128), (48, 384), (8192, 5120)])
def test_tile_int4_equals_tiled_quantizer(rows, K, group):
    """moe_quantize_int4 then moe_tile_int4 gives the bytes of moe_quantize_int4_tiled."""
    say(f"tile int4: rows={rows} K={K} group={group}")
    g = torch.Generator(device=DEV)
    g.manual_seed(rows * 31 + K + group)
    w = torch.randn(rows, K, device=DEV, generator=g) * 0.02
    w[1::9] *= 1e-5
    q_rm, s_rm = moe.quantize_int4(w, group=group)
    q_t, s_t = moe.tile_int4(q_rm, s_rm, group)
    q_ref, s_ref = moe.quantize_int4(w, tiled=True, group=group)
    torch.cuda.synchronize()
    assert torch.equal(q_t, q_ref)
    assert torch.equal(s_t.view(torch.int32), s_ref.view(torch.int32))


def _experts_two_ways(cfg, group=128):
    """The layer's routed experts quantized row-major and repacked, and tiled directly."""
    a = moe.Int4Experts.empty(cfg.E, cfg.d, cfg.h, DEV, group)
    b = moe.Int4Experts.empty(cfg.E, cfg.d, cfg.h, DEV, group)
    for e in range(cfg.E):
        ws = [W.gen_expert_weight(cfg, n, e, DEV) for n in ("w1", "w3", "w2")]
        parts = []
        for w in ws:
            parts.extend(moe.quantize_int4(w, group=group))
        a.set_expert_rowmajor(e, *parts)
        b.quantize_expert(e, *ws)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("i,group", [(0, 128), (0, 32), (1, 128), (2, 128)])
def test_rowmajor_quantizer_feeds_the_forward(i, group):
    """moe_quantize_int4 -> moe_tile_int4 -> moe_forward equals
    moe_quantize_int4_tiled -> moe_forward bit for bit."""
    cfg = W.config(i)
    say(f"row-major experts through moe_tile_int4: config {i} ({cfg.name}) group {group}")
    a, b = _experts_two_ways(cfg, group)
    for name in ("w1q", "w3q", "w2q", "w1s", "w3s", "w2s"):
        assert torch.equal(getattr(a, name).view(torch.uint8), getattr(b, name).view(torch.uint8)), name
    x = W.gen_x(cfg).to(DEV)
    wr, bias = W.gen_router(cfg)
    wr = wr.to(DEV)
    bias = None if bias is None else bias.to(DEV)
    shared = moe.pack_shared(*(s.to(DEV) for s in W.gen_shared(cfg, DEV)))
    ya = moe.forward(x, wr, bias, a, shared, cfg.top_k)
    yb = moe.forward(x, wr, bias, b, shared, cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))

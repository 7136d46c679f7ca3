"""The C ABI library on the host, no GPU needed.

* it loads and exports every function include/moe_int4.h declares;
* every validation error returns before any HIP call, with the right code
  and a detail string (pointers here are never dereferenced);
* workspace sizing.
"""
import ctypes
import os
import re

import pytest

import moe_ffn_int4_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_int4.h")

OK, INVALID, UNSUPPORTED, HIPERR, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x10000  # an aligned, never-dereferenced address


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from moe_ffn_int4_amd import build
        build.build()
    return moe.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for need in ("moe_quantize_int4", "moe_quantize_int4_tiled", "moe_tile_int4", "moe_pack_bf16_tiled",
                 "moe_forward", "moe_forward_path", "moe_route",
                 "moe_forward_workspace_bytes", "moe_route_workspace_bytes",
                 "moe_status_string", "moe_last_error", "moe_abi_version", "moe_device_check"):
        assert need in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), f"{name} not exported"
    assert L.moe_abi_version() == 1


def test_status_strings(L):
    for code in (OK, INVALID, UNSUPPORTED, HIPERR, WORKSPACE, 99):
        assert L.moe_status_string(code)


def _dims(T=64, d=256, E=4, h=512, k=1, g=128):
    return moe._Dims(T, d, E, h, k, g)


def _call_forward(L, dims, x=FAKE, wr=FAKE, b=None, experts=None, shared=None, y=FAKE,
                  path=0, ws=FAKE * 16, ws_bytes=None):
    if experts is None:
        experts = moe._Experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    if shared is None:
        shared = moe._Shared(FAKE, FAKE, FAKE)
    if ws_bytes is None:
        ws_bytes = L.moe_forward_workspace_bytes(ctypes.byref(dims)) or (1 << 40)
    return L.moe_forward_path(ctypes.byref(dims), x, wr, b, ctypes.byref(experts),
                              ctypes.byref(shared), y, None, None, path, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(T=0), "T = 0"),
    (dict(d=100), "d = 100"),
    (dict(h=200), "h = 200"),
    (dict(E=0), "E = 0"),
    (dict(E=300), "E = 300"),
    (dict(k=0), "top_k = 0"),
    (dict(E=4, k=5), "top_k = 5"),
    (dict(E=32, k=17), "top_k = 17"),
    (dict(g=16), "group_size 16"),
    (dict(g=96), "group_size 96"),
])
def test_invalid_dims(L, kw, needle):
    assert _call_forward(L, _dims(**kw), ws_bytes=1 << 40) == INVALID
    assert needle in L.moe_last_error().decode()
    assert L.moe_forward_workspace_bytes(ctypes.byref(_dims(**kw))) == 0


@pytest.mark.parametrize("field", ["x", "wr", "y"])
def test_null_pointers(L, field):
    assert _call_forward(L, _dims(), **{field: None}) == INVALID
    assert "NULL" in L.moe_last_error().decode()


def test_null_expert_and_shared_fields(L):
    ex = moe._Experts(FAKE, FAKE, None, FAKE, FAKE, FAKE)
    assert _call_forward(L, _dims(), experts=ex) == INVALID
    assert "w2q" in L.moe_last_error().decode()
    sh = moe._Shared(FAKE, None, FAKE)
    assert _call_forward(L, _dims(), shared=sh) == INVALID
    assert "s3" in L.moe_last_error().decode()


def test_misaligned_pointer(L):
    assert _call_forward(L, _dims(), x=FAKE + 2) == INVALID
    assert "aligned" in L.moe_last_error().decode()


def test_unknown_path(L):
    assert _call_forward(L, _dims(), path=7) == INVALID


def test_workspace_errors(L):
    dims = _dims()
    need = L.moe_forward_workspace_bytes(ctypes.byref(dims))
    assert need > 0
    assert _call_forward(L, dims, ws=None) == WORKSPACE
    assert _call_forward(L, dims, ws_bytes=need - 1) == WORKSPACE
    assert "needs" in L.moe_last_error().decode()
    assert _call_forward(L, dims, ws=FAKE + 16) == WORKSPACE
    rneed = L.moe_route_workspace_bytes(ctypes.byref(dims))
    assert 0 < rneed < need


def test_workspace_grows_with_the_layer(L):
    small = L.moe_forward_workspace_bytes(ctypes.byref(_dims(T=64)))
    big = L.moe_forward_workspace_bytes(ctypes.byref(_dims(T=4096)))
    wide = L.moe_forward_workspace_bytes(ctypes.byref(_dims(T=4096, k=4)))
    assert small < big < wide
    # the wide-routing layer: H and O hold (T*k + T) rows
    d = moe._Dims(16384, 5120, 128, 8192, 8, 128)
    n = L.moe_forward_workspace_bytes(ctypes.byref(d))
    assert n >= (131072 + 16384) * (8192 * 2 + 5120 * 4)


def test_quantize_validation(L):
    assert L.moe_quantize_int4(FAKE, 4, 100, 128, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_int4(FAKE, 4, 256, 16, FAKE, FAKE, None) == INVALID
    assert "group_size 16" in L.moe_last_error().decode()
    assert L.moe_quantize_int4(FAKE, 4, 64, 32, FAKE, FAKE, None) == INVALID  # K % 128
    assert L.moe_quantize_int4(FAKE, 0, 256, 64, FAKE, FAKE, None) == OK
    assert L.moe_quantize_int4(FAKE, 0, 256, 32, FAKE, FAKE, None) == OK
    assert L.moe_quantize_int4(FAKE, -1, 256, 128, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_int4(None, 4, 256, 128, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_int4(FAKE, 4, 256, 128, None, FAKE, None) == INVALID
    assert L.moe_quantize_int4(FAKE, 4, 256, 128, FAKE, FAKE + 1, None) == INVALID
    assert L.moe_quantize_int4(FAKE, 4, 256, 128, FAKE + 8, FAKE, None) == INVALID  # q 16-byte aligned
    assert "aligned" in L.moe_last_error().decode()
    assert L.moe_quantize_int4(FAKE, 0, 256, 128, FAKE, FAKE, None) == OK  # nothing to do


def test_tile_int4_validation(L):
    A, B, C, D = FAKE, FAKE * 64, FAKE * 128, FAKE * 192  # far apart: no overlap
    assert L.moe_tile_int4(A, B, 20, 256, 128, C, D, None) == INVALID
    assert "multiple of 16" in L.moe_last_error().decode()
    assert L.moe_tile_int4(A, B, 32, 200, 128, C, D, None) == INVALID
    assert L.moe_tile_int4(A, B, 32, 256, 16, C, D, None) == INVALID
    assert "group_size" in L.moe_last_error().decode()
    assert L.moe_tile_int4(None, B, 32, 256, 128, C, D, None) == INVALID
    assert L.moe_tile_int4(A + 8, B, 32, 256, 128, C, D, None) == INVALID
    assert L.moe_tile_int4(A, B + 2, 32, 256, 128, C, D, None) == INVALID
    assert L.moe_tile_int4(A, B, 32, 256, 128, None, D, None) == INVALID
    # 32 rows x 256 columns: 4 KB of codes; a tiled copy 1 KB further overlaps
    assert L.moe_tile_int4(A, B, 32, 256, 128, A + 1024, D, None) == INVALID
    assert "overlap" in L.moe_last_error().decode()
    assert L.moe_tile_int4(A, B, 32, 256, 128, C, B + 16, None) == INVALID
    assert L.moe_tile_int4(A, B, 0, 256, 128, C, D, None) == OK  # nothing to do


def test_tiled_quantize_and_pack_validation(L):
    assert L.moe_quantize_int4_tiled(FAKE, 20, 256, 128, FAKE, FAKE, None) == INVALID
    assert "multiple of 16" in L.moe_last_error().decode()
    assert L.moe_quantize_int4_tiled(FAKE, 32, 200, 128, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_int4_tiled(FAKE, 32, 256, 128, FAKE + 4, FAKE, None) == INVALID
    assert L.moe_quantize_int4_tiled(FAKE, 0, 256, 128, FAKE, FAKE, None) == OK
    assert L.moe_pack_bf16_tiled(FAKE, 16, 100, FAKE * 64, None) == INVALID
    assert L.moe_pack_bf16_tiled(FAKE, 17, 128, FAKE * 64, None) == INVALID
    assert L.moe_pack_bf16_tiled(FAKE, 16, 128, FAKE + 64, None) == INVALID  # overlap
    assert "overlap" in L.moe_last_error().decode()
    assert L.moe_pack_bf16_tiled(None, 16, 128, FAKE, None) == INVALID
    assert L.moe_pack_bf16_tiled(FAKE, 0, 128, FAKE, None) == OK


def test_route_validation(L):
    dims = _dims()
    n = L.moe_route_workspace_bytes(ctypes.byref(dims))
    assert L.moe_route(ctypes.byref(dims), FAKE, FAKE, None, None, FAKE, None, None, None, None,
                       None, FAKE * 16, n, None) == INVALID
    assert L.moe_route(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, None, None, None, None,
                       None, FAKE * 16, n - 1, None) == WORKSPACE


def test_valid_call_without_a_gpu_reports_the_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case is about hosts without one")
    assert _call_forward(L, _dims()) in (HIPERR, UNSUPPORTED)
    assert L.moe_device_check() in (HIPERR, UNSUPPORTED)


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.quantize_int4(torch.zeros(4, 128))


# ---- fp8 and bf16 routed experts, group sizes, paths (validation only)

def _call_fp8(L, dims, experts=None, ws_bytes=None, path=0, ub=0.0):
    if experts is None:
        experts = moe._ExpertsFp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ub)
    shared = moe._Shared(FAKE, FAKE, FAKE)
    if ws_bytes is None:
        ws_bytes = L.moe_forward_fp8_workspace_bytes(ctypes.byref(dims)) or (1 << 40)
    return L.moe_forward_fp8(ctypes.byref(dims), FAKE, FAKE, None, ctypes.byref(experts),
                             ctypes.byref(shared), FAKE, None, None, path, FAKE * 16, ws_bytes, None)


def test_fp8_workspace_is_larger_by_the_quantized_rows(L):
    d = _dims(T=64, d=256, E=4, h=512, k=2)
    base = L.moe_forward_workspace_bytes(ctypes.byref(d))
    fp8 = L.moe_forward_fp8_workspace_bytes(ctypes.byref(d))
    # x_q [T, d] + H_q [P, h] bytes and their fp32 row scales, each section 256-byte aligned
    assert fp8 - base >= 64 * 256 + 128 * 512 + 64 * 4 + 128 * 4
    assert L.moe_forward_fp8_workspace_bytes(ctypes.byref(_dims(T=0))) == 0


def test_fp8_forward_validation(L):
    d = _dims()
    ex = moe._ExpertsFp8(FAKE, FAKE, None, FAKE, FAKE, FAKE, 1200.0)
    assert _call_fp8(L, d, experts=ex) == INVALID
    assert "w2q" in L.moe_last_error().decode()
    for bad in (float("nan"), -1.0, float("inf")):
        assert _call_fp8(L, d, ub=bad) == INVALID
        assert "act_ub" in L.moe_last_error().decode()
    need = L.moe_forward_fp8_workspace_bytes(ctypes.byref(d))
    assert _call_fp8(L, d, ws_bytes=L.moe_forward_workspace_bytes(ctypes.byref(d))) == WORKSPACE
    assert need > L.moe_forward_workspace_bytes(ctypes.byref(d))
    assert _call_fp8(L, d, path=5) == INVALID
    assert "path" in L.moe_last_error().decode()
    null = L.moe_forward_fp8(ctypes.byref(d), FAKE, FAKE, None, None, ctypes.byref(moe._Shared(FAKE, FAKE, FAKE)),
                             FAKE, None, None, 0, FAKE * 16, need, None)
    assert null == INVALID and "experts" in L.moe_last_error().decode()


def test_bf16_forward_validation(L):
    d = _dims()
    ex = moe._ExpertsBf16(FAKE, None, FAKE)
    r = L.moe_forward_bf16(ctypes.byref(d), FAKE, FAKE, None, ctypes.byref(ex),
                           ctypes.byref(moe._Shared(FAKE, FAKE, FAKE)), FAKE, None, None, 0, FAKE * 16,
                           L.moe_forward_workspace_bytes(ctypes.byref(d)), None)
    assert r == INVALID and "w3" in L.moe_last_error().decode()


@pytest.mark.parametrize("g", [128, 64, 32])
def test_supported_group_sizes_pass_dims_validation(L, g):
    assert L.moe_forward_workspace_bytes(ctypes.byref(_dims(g=g))) > 0


def test_paths(L):
    for p in (0, 1, 2, 3, 4):
        # validation passes for every known path; without a GPU the device check fails next
        assert _call_forward(L, _dims(), path=p) in (HIPERR, UNSUPPORTED, OK)
    assert _call_forward(L, _dims(), path=5) == INVALID


def test_binding_group_sizes():
    import torch
    ex = moe.Int4Experts(*(torch.empty(s, dtype=dt) for s, dt in [
        ((2, 256, 64), torch.uint8), ((2, 256, 64), torch.uint8), ((2, 128, 128), torch.uint8),
        ((2, 256, 4), torch.float32), ((2, 256, 4), torch.float32), ((2, 128, 8), torch.float32)]))
    assert ex.group == 32 and ex.d == 128 and ex.h == 256
    with pytest.raises(ValueError):
        moe.Int4Experts.empty(2, 128, 256, "cpu", group=48)
    t = torch.arange(32 * 4, dtype=torch.float32)
    s = moe.untile_scales(t, 32, 256, 64)  # tiled (t*16 + row)*S + s  ->  row-major [rows, K/g]
    assert s.shape == (32, 4)
    # row 17, group 3: tile (1, 1), row 1, scale 1 of that tile -> ((1*2+1)*16 + 1)*2 + 1
    assert s[17, 3].item() == ((1 * 2 + 1) * 16 + 1) * 2 + 1


def test_noalloc_validation(L):
    """moe_forward_noalloc refuses bad dims and layers past its scratch before any HIP call."""
    ex = ctypes.byref(moe._Experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    sh = ctypes.byref(moe._Shared(FAKE, FAKE, FAKE))
    bad = _dims(T=0)
    assert L.moe_forward_noalloc(ctypes.byref(bad), FAKE, FAKE, None, ex, sh, FAKE, None, None,
                                 0, None) == INVALID
    assert L.moe_forward_noalloc(ctypes.byref(_dims()), FAKE, FAKE, None, None, sh, FAKE, None,
                                 None, 0, None) == INVALID
    big = moe._Dims(8192, 5120, 16, 8192, 1, 128)
    assert L.moe_forward_workspace_bytes(ctypes.byref(big)) > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big), FAKE, FAKE, None, ex, sh, FAKE, None, None,
                                 0, None) == WORKSPACE
    assert "MOE_NOALLOC_SCRATCH_BYTES" in L.moe_last_error().decode()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)" in open(HEADER).read()
    assert moe.NOALLOC_SCRATCH_BYTES == 64 << 20

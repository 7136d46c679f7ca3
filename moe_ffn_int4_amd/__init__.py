"""MI355X (gfx950) int4 Mixture-of-Experts feed-forward layer.

Thin ctypes binding over ``libmoe_int4.so`` (C ABI in ``include/moe_int4.h``).
This module only checks and marshals arguments: torch provides device memory
and the current HIP stream, and every step of the layer runs in the library's
HIP kernels. There is no fallback: if the library is missing, importing the
functions below raises.

    q, s = quantize_int4(w_fp32_cuda)                 # int4 group quantizer
    experts = Int4Experts.empty(E, d, h, dev)         # routed experts, tiled int4
    experts.quantize_expert(e, w1, w3, w2)            #   (fp32 weights on the GPU)
    shared = pack_shared(s1, s3, s2)                  # shared expert, tiled bf16
    y = forward(x, router_w, router_b, experts, shared, top_k)
    r = route(x, router_w, router_b, top_k)           # routing/dispatch only

Weights live in the tiled layouts the kernels read (see include/moe_int4.h);
untile_int4 / untile_scales / untile_bf16 convert them back to row-major.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_int4.so")
GROUP = 128                 # default int4 quantization group
GROUPS = (128, 64, 32)      # supported int4 groups (weights per scale)
TILE = 128                  # columns of a weight tile
PATHS = {"auto": 0, "prefill": 1, "decode": 2, "hybrid": 3, "prefill_wide": 4}

MOE_OK = 0


class MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_string(status)} [{status}]: {detail}")


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
                ("h", ctypes.c_int64), ("top_k", ctypes.c_int32), ("group_size", ctypes.c_int32)]


class _Experts(ctypes.Structure):
    _fields_ = [("w1q", ctypes.c_void_p), ("w3q", ctypes.c_void_p), ("w2q", ctypes.c_void_p),
                ("w1s", ctypes.c_void_p), ("w3s", ctypes.c_void_p), ("w2s", ctypes.c_void_p)]


class _Shared(ctypes.Structure):
    _fields_ = [("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


class _ExpertsBf16(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class _ExpertsFp8(ctypes.Structure):
    _fields_ = [("w1q", ctypes.c_void_p), ("w3q", ctypes.c_void_p), ("w2q", ctypes.c_void_p),
                ("w1s", ctypes.c_void_p), ("w3s", ctypes.c_void_p), ("w2s", ctypes.c_void_p),
                ("act_ub", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m moe_ffn_int4_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_device_check.restype = ctypes.c_int
        L.moe_hbm_read.argtypes = [P, i64, P, P]
        L.moe_hbm_read.restype = ctypes.c_int
        L.moe_hbm_read_sink_words.restype = ctypes.c_int
        L.moe_hbm_copy.argtypes = [P, P, i64, P]
        L.moe_hbm_copy.restype = ctypes.c_int
        L.moe_quantize_int4.argtypes = [P, i64, i64, i32, P, P, P]
        L.moe_quantize_int4.restype = ctypes.c_int
        L.moe_quantize_int4_tiled.argtypes = [P, i64, i64, i32, P, P, P]
        L.moe_quantize_int4_tiled.restype = ctypes.c_int
        L.moe_tile_int4.argtypes = [P, P, i64, i64, i32, P, P, P]
        L.moe_tile_int4.restype = ctypes.c_int
        L.moe_pack_bf16_tiled.argtypes = [P, i64, i64, P, P]
        L.moe_pack_bf16_tiled.restype = ctypes.c_int
        L.moe_forward_workspace_bytes.argtypes = [ctypes.POINTER(_Dims)]
        L.moe_forward_workspace_bytes.restype = sz
        fwd = [ctypes.POINTER(_Dims), P, P, P, ctypes.POINTER(_Experts), ctypes.POINTER(_Shared),
               P, P, P]
        L.moe_forward.argtypes = fwd + [P, sz, P]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_path.argtypes = fwd + [i32, P, sz, P]
        L.moe_forward_path.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = fwd + [i32, P]
        L.moe_forward_noalloc.restype = ctypes.c_int
        fwd_bf16 = list(fwd)
        fwd_bf16[4] = ctypes.POINTER(_ExpertsBf16)
        L.moe_forward_bf16.argtypes = fwd_bf16 + [i32, P, sz, P]
        fwd_fp8 = list(fwd)
        fwd_fp8[4] = ctypes.POINTER(_ExpertsFp8)
        L.moe_forward_fp8.argtypes = fwd_fp8 + [i32, P, sz, P]
        L.moe_forward_fp8.restype = ctypes.c_int
        L.moe_forward_fp8_workspace_bytes.argtypes = [ctypes.POINTER(_Dims)]
        L.moe_forward_fp8_workspace_bytes.restype = sz
        L.moe_quantize_fp8_tiled.argtypes = [P, i64, i64, P, P, P]
        L.moe_quantize_fp8_tiled.restype = ctypes.c_int
        L.moe_quantize_fp8_rows.argtypes = [P, i64, i64, ctypes.c_float, P, P, P]
        L.moe_quantize_fp8_rows.restype = ctypes.c_int
        L.moe_forward_bf16.restype = ctypes.c_int
        L.moe_route_workspace_bytes.argtypes = [ctypes.POINTER(_Dims)]
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.moe_route.restype = ctypes.c_int
        L.moe_profile_enable.argtypes = [ctypes.c_int]
        L.moe_profile_enable.restype = ctypes.c_int
        L.moe_profile_read.argtypes = [P, P, ctypes.c_int]
        L.moe_profile_read.restype = ctypes.c_int
        L.moe_stage_name.argtypes = [ctypes.c_int]
        L.moe_stage_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(T, d, E, h, top_k, group: int = GROUP) -> _Dims:
    return _Dims(int(T), int(d), int(E), int(h), int(top_k), int(group))


# --------------------------------------------------------------- quantizer

def quantize_int4(w: torch.Tensor, q: Optional[torch.Tensor] = None,
                  scales: Optional[torch.Tensor] = None, tiled: bool = False,
                  group: int = GROUP):
    """Int4 group quantizer: fp32 [rows, K] -> (uint8 [rows, K/2], fp32 [rows, K/group]).

    ``w`` may have leading batch dims; they are flattened into rows. With
    ``tiled`` the outputs hold the same codes and scales in the 16-row tile
    order the forward pass reads (rows must be a multiple of 16). ``group``:
    128, 64 or 32 weights per scale (K a multiple of 128).
    """
    _need(w, "w", torch.float32)
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if q is None:
        q = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(w.shape[:-1] + (K // group,), dtype=torch.float32, device=w.device)
    _need(q, "q", torch.uint8)
    _need(scales, "scales", torch.float32)
    if q.numel() != rows * (K // 2) or scales.numel() != rows * (K // group):
        raise ValueError("q / scales have the wrong number of elements")
    fn = lib().moe_quantize_int4_tiled if tiled else lib().moe_quantize_int4
    _check(fn(_ptr(w), rows, K, int(group), _ptr(q), _ptr(scales), _stream(w.device)))
    return q, scales


def tile_int4(q: torch.Tensor, scales: torch.Tensor, group: int = GROUP,
              q_tiled: Optional[torch.Tensor] = None,
              scales_tiled: Optional[torch.Tensor] = None):
    """Row-major int4 (``quantize_int4`` output: uint8 [rows, K/2] and fp32
    [rows, K/group]) -> the tiled order the forward pass reads (same shapes)."""
    _need(q, "q", torch.uint8)
    _need(scales, "scales", torch.float32)
    if q.dim() != 2 or scales.dim() != 2:
        raise ValueError("q and scales must be 2-D")
    rows, K = q.shape[0], q.shape[1] * 2
    if tuple(scales.shape) != (rows, K // group):
        raise ValueError(f"scales has shape {tuple(scales.shape)}, expected {(rows, K // group)}")
    if q_tiled is None:
        q_tiled = torch.empty_like(q)
    if scales_tiled is None:
        scales_tiled = torch.empty_like(scales)
    _need(q_tiled, "q_tiled", torch.uint8)
    _need(scales_tiled, "scales_tiled", torch.float32)
    if q_tiled.numel() != q.numel() or scales_tiled.numel() != scales.numel():
        raise ValueError("q_tiled / scales_tiled have the wrong number of elements")
    _check(lib().moe_tile_int4(_ptr(q), _ptr(scales), rows, K, int(group), _ptr(q_tiled),
                               _ptr(scales_tiled), _stream(q.device)))
    return q_tiled, scales_tiled


def pack_bf16_tiled(src: torch.Tensor, dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [rows, K] -> the tiled order the forward pass reads (same shape)."""
    _need(src, "src", torch.bfloat16)
    if src.dim() != 2:
        raise ValueError("src must be 2-D")
    rows, K = src.shape
    if dst is None:
        dst = torch.empty_like(src)
    _need(dst, "dst", torch.bfloat16, (rows, K))
    _check(lib().moe_pack_bf16_tiled(_ptr(src), rows, K, _ptr(dst), _stream(src.device)))
    return dst


def quantize_fp8(w: torch.Tensor, q: Optional[torch.Tensor] = None,
                 scales: Optional[torch.Tensor] = None):
    """fp32 weights [rows, K] -> fp8 E4M3 codes (uint8, tiled order) and fp32 row scales."""
    _need(w, "w", torch.float32)
    rows, K = w.shape
    if q is None:
        q = torch.empty(rows, K, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=w.device)
    _need(q, "q", torch.uint8, (rows, K))
    _need(scales, "scales", torch.float32, (rows,))
    _check(lib().moe_quantize_fp8_tiled(_ptr(w), rows, K, _ptr(q), _ptr(scales), _stream(w.device)))
    return q, scales


def quantize_fp8_rows(x: torch.Tensor, ub: float):
    """bf16 activations [rows, K] -> row-major fp8 codes and fp32 row scales
    (the row maximum bounded by ``ub``; ``ub <= 0``: no bound)."""
    _need(x, "x", torch.bfloat16)
    rows, K = x.shape
    q = torch.empty(rows, K, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib().moe_quantize_fp8_rows(_ptr(x), rows, K, float(ub), _ptr(q), _ptr(scales),
                                       _stream(x.device)))
    return q, scales


def untile_fp8(q: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    """Tiled fp8 codes back to row-major [rows, K] (CPU or GPU tensor)."""
    t = q.reshape(rows // 16, K // 128, 4, 16, 32)  # row tile, k tile, step, row, column
    return t.permute(0, 3, 1, 2, 4).reshape(rows, K)


def pack_shared(s1: torch.Tensor, s3: torch.Tensor, s2: torch.Tensor):
    """The shared expert's bf16 weights (S1, S3 [h, d], S2 [d, h]) in tiled order."""
    return tuple(pack_bf16_tiled(s) for s in (s1, s3, s2))


@dataclass
class Int4Experts:
    """Stacked routed experts in the library's int4 layout."""

    w1q: torch.Tensor  # uint8 [E, h, d/2]
    w3q: torch.Tensor  # uint8 [E, h, d/2]
    w2q: torch.Tensor  # uint8 [E, d, h/2]
    w1s: torch.Tensor  # fp32  [E, h, d/group]
    w3s: torch.Tensor  # fp32  [E, h, d/group]
    w2s: torch.Tensor  # fp32  [E, d, h/group]

    @property
    def E(self) -> int:
        return self.w1q.shape[0]

    @property
    def h(self) -> int:
        return self.w1q.shape[1]

    @property
    def d(self) -> int:
        return self.w2q.shape[1]

    @property
    def group(self) -> int:
        """Weights per scale (128, 64 or 32)."""
        return self.d // self.w1s.shape[2]

    @staticmethod
    def empty(E: int, d: int, h: int, device, group: int = GROUP) -> "Int4Experts":
        if group not in GROUPS:
            raise ValueError(f"group {group} unsupported {GROUPS}")
        u8, f32 = torch.uint8, torch.float32
        return Int4Experts(
            torch.empty(E, h, d // 2, dtype=u8, device=device),
            torch.empty(E, h, d // 2, dtype=u8, device=device),
            torch.empty(E, d, h // 2, dtype=u8, device=device),
            torch.empty(E, h, d // group, dtype=f32, device=device),
            torch.empty(E, h, d // group, dtype=f32, device=device),
            torch.empty(E, d, h // group, dtype=f32, device=device))

    def quantize_expert(self, e: int, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor):
        """Quantize one expert's fp32 weights (on the GPU) into slot ``e`` (tiled)."""
        g = self.group
        quantize_int4(w1, self.w1q[e], self.w1s[e], tiled=True, group=g)
        quantize_int4(w3, self.w3q[e], self.w3s[e], tiled=True, group=g)
        quantize_int4(w2, self.w2q[e], self.w2s[e], tiled=True, group=g)

    def set_expert_rowmajor(self, e: int, q1, s1, q3, s3, q2, s2):
        """Slot ``e`` from row-major int4 (``quantize_int4`` without ``tiled``):
        W1, W3 codes [h, d/2] and scales [h, d/group], W2 [d, h/2] and [d, h/group],
        repacked into the tiled order by ``tile_int4``."""
        g = self.group
        tile_int4(q1, s1, g, self.w1q[e], self.w1s[e])
        tile_int4(q3, s3, g, self.w3q[e], self.w3s[e])
        tile_int4(q2, s2, g, self.w2q[e], self.w2s[e])

    def _struct(self) -> _Experts:
        for name in ("w1q", "w3q", "w2q"):
            _need(getattr(self, name), name, torch.uint8)
        for name in ("w1s", "w3s", "w2s"):
            _need(getattr(self, name), name, torch.float32)
        g = self.group
        if (g not in GROUPS or self.w1s.shape[2] * g != self.d or self.w3s.shape != self.w1s.shape
                or self.w2s.shape[2] * g != self.h):
            raise ValueError("int4 scales do not match one of the supported groups")
        return _Experts(*(getattr(self, n).data_ptr() for n in
                          ("w1q", "w3q", "w2q", "w1s", "w3s", "w2s")))


# ----------------------------------------------------------------- forward

def workspace_bytes(T: int, d: int, E: int, h: int, top_k: int, fp8: bool = False) -> int:
    """Workspace bytes of the forward (``fp8``: with fp8 routed experts)."""
    dims = _dims(T, d, E, h, top_k)
    fn = lib().moe_forward_fp8_workspace_bytes if fp8 else lib().moe_forward_workspace_bytes
    n = fn(ctypes.byref(dims))
    if n == 0:
        raise ValueError(f"invalid layer dims T={T} d={d} E={E} h={h} top_k={top_k}")
    return n


def alloc_workspace(T: int, d: int, E: int, h: int, top_k: int, device,
                    fp8: bool = False) -> torch.Tensor:
    return torch.empty(workspace_bytes(T, d, E, h, top_k, fp8), dtype=torch.uint8, device=device)


@dataclass
class Bf16Experts:
    """Stacked routed experts in bf16 (the pure-bf16 baseline path), each matrix in
    the tiled order of ``pack_bf16_tiled``."""

    w1: torch.Tensor  # bf16 [E, h, d]
    w3: torch.Tensor  # bf16 [E, h, d]
    w2: torch.Tensor  # bf16 [E, d, h]

    @property
    def E(self) -> int:
        return self.w1.shape[0]

    @property
    def h(self) -> int:
        return self.w1.shape[1]

    @property
    def d(self) -> int:
        return self.w2.shape[1]

    @staticmethod
    def empty(E: int, d: int, h: int, device) -> "Bf16Experts":
        b = torch.bfloat16
        return Bf16Experts(torch.empty(E, h, d, dtype=b, device=device),
                           torch.empty(E, h, d, dtype=b, device=device),
                           torch.empty(E, d, h, dtype=b, device=device))

    def set_expert(self, e: int, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor):
        """Pack one expert's bf16 weights (W1, W3 [h, d], W2 [d, h]) into slot ``e``."""
        pack_bf16_tiled(w1, self.w1[e])
        pack_bf16_tiled(w3, self.w3[e])
        pack_bf16_tiled(w2, self.w2[e])

    def _struct(self) -> _ExpertsBf16:
        for name in ("w1", "w3", "w2"):
            _need(getattr(self, name), name, torch.bfloat16)
        return _ExpertsBf16(self.w1.data_ptr(), self.w3.data_ptr(), self.w2.data_ptr())


@dataclass
class Fp8Experts:
    """Stacked routed experts in fp8 E4M3 with one fp32 scale per weight row (the
    fp8_mixed path), codes in the tiled order of ``quantize_fp8``; ``act_ub`` bounds
    the activation row scales."""

    w1q: torch.Tensor  # uint8 [E, h, d]
    w3q: torch.Tensor  # uint8 [E, h, d]
    w2q: torch.Tensor  # uint8 [E, d, h]
    w1s: torch.Tensor  # fp32  [E, h]
    w3s: torch.Tensor  # fp32  [E, h]
    w2s: torch.Tensor  # fp32  [E, d]
    act_ub: float

    @property
    def E(self) -> int:
        return self.w1q.shape[0]

    @property
    def h(self) -> int:
        return self.w1q.shape[1]

    @property
    def d(self) -> int:
        return self.w2q.shape[1]

    @staticmethod
    def empty(E: int, d: int, h: int, device, act_ub: float) -> "Fp8Experts":
        u8, f32 = torch.uint8, torch.float32
        return Fp8Experts(
            torch.empty(E, h, d, dtype=u8, device=device),
            torch.empty(E, h, d, dtype=u8, device=device),
            torch.empty(E, d, h, dtype=u8, device=device),
            torch.empty(E, h, dtype=f32, device=device),
            torch.empty(E, h, dtype=f32, device=device),
            torch.empty(E, d, dtype=f32, device=device),
            float(act_ub))

    def quantize_expert(self, e: int, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor):
        """Quantize one expert's fp32 weights (on the GPU) into slot ``e`` (tiled)."""
        quantize_fp8(w1, self.w1q[e], self.w1s[e])
        quantize_fp8(w3, self.w3q[e], self.w3s[e])
        quantize_fp8(w2, self.w2q[e], self.w2s[e])

    def _struct(self) -> _ExpertsFp8:
        for name in ("w1q", "w3q", "w2q"):
            _need(getattr(self, name), name, torch.uint8)
        for name in ("w1s", "w3s", "w2s"):
            _need(getattr(self, name), name, torch.float32)
        return _ExpertsFp8(*(getattr(self, n).data_ptr() for n in
                             ("w1q", "w3q", "w2q", "w1s", "w3s", "w2s")), float(self.act_ub))


def forward(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor],
            experts, shared, top_k: int, path: str = "auto",
            y: Optional[torch.Tensor] = None, topk_ids: Optional[torch.Tensor] = None,
            topk_gates: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The MoE layer: y bf16 [T, d]. ``experts``: ``Int4Experts``, ``Bf16Experts`` or
    ``Fp8Experts``;
    ``shared`` = (S1 [h, d], S3 [h, d], S2 [d, h]) bf16, packed by ``pack_shared``."""
    _need(x, "x", torch.bfloat16)
    T, d = x.shape
    E, h = router_w.shape[0], experts.h
    _need(router_w, "router_w", torch.float32, (E, d))
    if router_b is not None:
        _need(router_b, "router_b", torch.float32, (E,))
    s1, s3, s2 = shared
    _need(s1, "S1", torch.bfloat16, (h, d))
    _need(s3, "S3", torch.bfloat16, (h, d))
    _need(s2, "S2", torch.bfloat16, (d, h))
    if experts.E != E or experts.d != d:
        raise ValueError("experts do not match the router / x")
    if y is None:
        y = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, (T, d))
    if topk_ids is not None:
        _need(topk_ids, "topk_ids", torch.int32, (T, top_k))
    if topk_gates is not None:
        _need(topk_gates, "topk_gates", torch.float32, (T, top_k))
    fp8 = isinstance(experts, Fp8Experts)
    if workspace is None:
        workspace = alloc_workspace(T, d, E, h, top_k, x.device, fp8)
    dims = _dims(T, d, E, h, top_k, experts.group if isinstance(experts, Int4Experts) else GROUP)
    ex = experts._struct()
    sh = _Shared(s1.data_ptr(), s3.data_ptr(), s2.data_ptr())
    if fp8:
        entry = lib().moe_forward_fp8
    elif isinstance(experts, Bf16Experts):
        entry = lib().moe_forward_bf16
    else:
        entry = lib().moe_forward_path
    _check(entry(
        ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b), ctypes.byref(ex),
        ctypes.byref(sh), _ptr(y), _ptr(topk_ids), _ptr(topk_gates), PATHS[path],
        _ptr(workspace), workspace.numel(), _stream(x.device)))
    return y


def forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor],
                    experts: "Int4Experts", shared, top_k: int, path: str = "auto",
                    y: Optional[torch.Tensor] = None, topk_ids: Optional[torch.Tensor] = None,
                    topk_gates: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``forward`` for int4 experts through the allocation-free entry point: its
    workspace is the library's static device scratch (NOALLOC_SCRATCH_BYTES),
    shared by every such call on the GPU, so overlapping calls race."""
    _need(x, "x", torch.bfloat16)
    T, d = x.shape
    E, h = router_w.shape[0], experts.h
    _need(router_w, "router_w", torch.float32, (E, d))
    if router_b is not None:
        _need(router_b, "router_b", torch.float32, (E,))
    s1, s3, s2 = shared
    _need(s1, "S1", torch.bfloat16, (h, d))
    _need(s3, "S3", torch.bfloat16, (h, d))
    _need(s2, "S2", torch.bfloat16, (d, h))
    if not isinstance(experts, Int4Experts) or experts.E != E or experts.d != d:
        raise ValueError("experts must be Int4Experts matching the router / x")
    if y is None:
        y = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, (T, d))
    if topk_ids is not None:
        _need(topk_ids, "topk_ids", torch.int32, (T, top_k))
    if topk_gates is not None:
        _need(topk_gates, "topk_gates", torch.float32, (T, top_k))
    dims = _dims(T, d, E, h, top_k, experts.group)
    ex = experts._struct()
    sh = _Shared(s1.data_ptr(), s3.data_ptr(), s2.data_ptr())
    _check(lib().moe_forward_noalloc(
        ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b), ctypes.byref(ex),
        ctypes.byref(sh), _ptr(y), _ptr(topk_ids), _ptr(topk_gates), PATHS[path],
        _stream(x.device)))
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20


def route(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor],
          top_k: int, workspace: Optional[torch.Tensor] = None) -> dict:
    """Routing and dispatch alone: ids, gates, logits, counts, offsets, perm, inv."""
    _need(x, "x", torch.bfloat16)
    T, d = x.shape
    E = router_w.shape[0]
    _need(router_w, "router_w", torch.float32, (E, d))
    if router_b is not None:
        _need(router_b, "router_b", torch.float32, (E,))
    dev = x.device
    P = T * top_k
    out = {
        "ids": torch.empty(T, top_k, dtype=torch.int32, device=dev),
        "gates": torch.empty(T, top_k, dtype=torch.float32, device=dev),
        "logits": torch.empty(T, E, dtype=torch.float32, device=dev),
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "perm": torch.empty(P, dtype=torch.int32, device=dev),
        "inv": torch.empty(P, dtype=torch.int32, device=dev),
    }
    dims = _dims(T, d, E, 128, top_k)
    if workspace is None:
        n = lib().moe_route_workspace_bytes(ctypes.byref(dims))
        if n == 0:
            raise ValueError(f"invalid routing dims T={T} d={d} E={E} top_k={top_k}")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(lib().moe_route(
        ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(out["ids"]),
        _ptr(out["gates"]), _ptr(out["logits"]), _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["perm"]), _ptr(out["inv"]), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def untile_int4(q: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    """Tiled int4 bytes of one [rows, K] matrix -> row-major bytes [rows, K/2]."""
    t = q.reshape(rows // 16, K // TILE, 4, 16, 16)  # row tile, k tile, step, row, byte
    return t.permute(0, 3, 1, 2, 4).reshape(rows, K // 2)


def untile_scales(s: torch.Tensor, rows: int, K: int, group: int = GROUP) -> torch.Tensor:
    """Tiled scales of one [rows, K] matrix -> row-major [rows, K/group]."""
    S = TILE // group
    return s.reshape(rows // 16, K // TILE, 16, S).permute(0, 2, 1, 3).reshape(rows, K // group)


def untile_bf16(t: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    """Tiled bf16 [rows, K] (pack_bf16_tiled order) -> row-major [rows, K]."""
    return t.reshape(rows // 16, K // TILE, 4, 16, 32).permute(0, 3, 1, 2, 4).reshape(rows, K)


def unpack_int4(q: torch.Tensor) -> torch.Tensor:
    """Packed bytes [..., K/2] -> int8 codes [..., K] (low nibble = even index)."""
    lo = (q.to(torch.int16) & 0xF)
    hi = (q.to(torch.int16) >> 4) & 0xF
    codes = torch.stack([lo, hi], dim=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    return torch.where(codes >= 8, codes - 16, codes).to(torch.int8)


# ------------------------------------------------------------------ timing

STAGE_COUNT = 10


def hbm_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream every 16-byte word of `buf` once (measurement helper); each block
    writes the XOR of the words it read into `sink` (uint32/int32,
    ``hbm_read_sink_words()`` entries)."""
    if not buf.is_cuda or not sink.is_cuda or sink.numel() < hbm_read_sink_words():
        raise ValueError("buf and sink must be device tensors, sink of hbm_read_sink_words() words")
    _check(lib().moe_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                              _stream(buf.device)))


def hbm_read_sink_words() -> int:
    return int(lib().moe_hbm_read_sink_words())


def hbm_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """Copy `src` into `dst` with the library's plain copy kernel (measurement helper)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not dst.is_cuda or not src.is_cuda:
        raise ValueError("dst and src must be device tensors of the same size")
    _check(lib().moe_hbm_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream(src.device)))


def profile_enable(on: bool = True) -> None:
    """Time each stage of later calls with events that its kernels record at
    their own start and end."""
    _check(lib().moe_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{stage name: (summed ms, launches)} since the last read; resets the sums."""
    ms = (ctypes.c_double * STAGE_COUNT)()
    n = (ctypes.c_int64 * STAGE_COUNT)()
    _check(lib().moe_profile_read(ms, n, STAGE_COUNT))
    return {lib().moe_stage_name(i).decode(): (ms[i], n[i]) for i in range(STAGE_COUNT)}

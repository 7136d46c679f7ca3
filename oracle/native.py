"""ctypes loader for the plain C oracle (test infrastructure only).

``build()`` compiles ``csrc/oracle.c`` with gcc (OpenMP, no fast-math, no FMA
contraction) into ``oracle/_build/liboracle.so``. The functions below only
marshal numpy arrays into the C loops; the arithmetic is in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Callable, Optional, Sequence, Union

import numpy as np

from .fp8 import Fp8Expert
from .moe import Bf16Expert, Int4Expert, MoEResult, _f64
from .quantize import GROUP

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle; returns the path of the shared library."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """The loaded C oracle (built on first use if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.oracle_quantize_int4.argtypes = [P, i64, i64, i64, P, P]
        L.oracle_quantize_int4.restype = None
        L.oracle_swiglu_int4_token.argtypes = [P, i64, i64, i64, P, P, P, P, P, P, P, P]
        L.oracle_swiglu_int4_token.restype = None
        L.oracle_swiglu_bf16_token.argtypes = [P, i64, i64, P, P, P, P, P]
        L.oracle_swiglu_bf16_token.restype = None
        L.oracle_router_token.argtypes = [P, P, P, i64, i64, P]
        L.oracle_router_token.restype = None
        L.oracle_topk_token.argtypes = [P, i64, i32, P]
        L.oracle_topk_token.restype = None
        L.oracle_moe_token.argtypes = ([P, i64, i64, i64, i32, i64, P, P]
                                       + [P] * 6 + [P] * 3 + [P] + [P] * 6)
        L.oracle_moe_token.restype = ctypes.c_int
        L.oracle_moe_token_bf16.argtypes = ([P, i64, i64, i64, i32, P, P]
                                            + [P] * 3 + [P] * 3 + [P] + [P] * 6)
        L.oracle_moe_token_bf16.restype = ctypes.c_int
        L.oracle_quantize_fp8_rows.argtypes = [P, i64, i64, ctypes.c_float, P, P]
        L.oracle_quantize_fp8_rows.restype = None
        L.oracle_fp8_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_value.restype = ctypes.c_double
        L.oracle_moe_token_fp8.argtypes = ([P, i64, i64, i64, i32, P, P]
                                           + [P] * 6 + [ctypes.c_float] + [P] * 3 + [P] + [P] * 8)
        L.oracle_moe_token_fp8.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def quantize_int4(w, group_size: int = GROUP):
    """C loop form of the quantizer: ``(codes int8, scales fp32)``."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    rows = w.size // K
    codes = np.empty(w.shape, dtype=np.int8)
    scales = np.empty(w.shape[:-1] + (K // group_size,), dtype=np.float32)
    lib().oracle_quantize_int4(_ptr(w), rows, K, group_size, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_fp8_rows(w, ub: Optional[float] = None):
    """C loop form of the fp8 row quantizer: ``(codes uint8, scales fp32 [rows])``;
    ``ub`` None or <= 0: no bound on the row scale."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    rows = w.size // K
    codes = np.empty(w.shape, dtype=np.uint8)
    scales = np.empty(w.shape[:-1], dtype=np.float32)
    lib().oracle_quantize_fp8_rows(_ptr(w), rows, K, 0.0 if ub is None else float(ub),
                                   _ptr(codes), _ptr(scales))
    return codes, scales


def fp8_expert(w1, w3, w2, ub: float) -> Fp8Expert:
    """An fp8 expert quantized by the C loops (same fields as ``Fp8Expert.from_fp32``)."""
    q1, s1 = quantize_fp8_rows(w1)
    q3, s3 = quantize_fp8_rows(w3)
    q2, s2 = quantize_fp8_rows(w2)
    return Fp8Expert(q1, s1, q3, s3, q2, s2, float(ub))


def _bf16_bits(a) -> np.ndarray:
    """uint16 bit patterns of a bf16 torch tensor (or pass uint16 through)."""
    if hasattr(a, "detach"):
        import torch
        return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy()
                                    .view(np.uint16))
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 weights must be a torch bf16 tensor or uint16 bits")
    return np.ascontiguousarray(a)


ExpertSource = Union[Sequence[Optional[Union[Int4Expert, Bf16Expert]]],
                     Callable[[int], Optional[Union[Int4Expert, Bf16Expert]]]]


def moe_forward_per_token(x, wr, b, top_k: int, experts: ExpertSource, shared,
                          forced_ids: Optional[np.ndarray] = None,
                          group_size: int = GROUP) -> MoEResult:
    """The layer as a per-token loop in C (pins the grouped numpy form).

    ``experts`` is a sequence (entries may be None for experts no token picks)
    or a callable ``e -> Int4Expert``; with a callable, every expert is fetched
    once up front, so pass a sequence for large layers.
    """
    xf = np.ascontiguousarray(_f64(x))
    T, d = xf.shape
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    E = wr.shape[0]
    bias = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    seq = [experts(e) for e in range(E)] if callable(experts) else list(experts)
    sh1, sh3, sh2 = (_bf16_bits(s) for s in shared)
    h = sh1.shape[0]

    def arr(field, dtype):
        a = (ctypes.c_void_p * E)()
        keep = []
        for e, ex in enumerate(seq):
            if ex is None:
                a[e] = None
            else:
                v = np.ascontiguousarray(getattr(ex, field), dtype=dtype)
                keep.append(v)
                a[e] = v.ctypes.data
        return a, keep

    kinds = {type(ex) for ex in seq if ex is not None}
    if len(kinds) > 1:
        raise TypeError("routed experts must all be of one kind (int4, bf16 or fp8)")
    bf16 = Bf16Expert in kinds
    fp8 = Fp8Expert in kinds
    if fp8:
        q1, k1 = arr("q1", np.uint8); s1, k2 = arr("s1", np.float32)
        q3, k3 = arr("q3", np.uint8); s3, k4 = arr("s3", np.float32)
        q2, k5 = arr("q2", np.uint8); s2, k6 = arr("s2", np.float32)
        keep = (k1, k2, k3, k4, k5, k6)  # noqa: F841  (keeps arrays alive)
        ubs = {float(ex.ub) for ex in seq if ex is not None}
        if len(ubs) > 1:
            raise ValueError("fp8 experts must share one activation scale bound")
        ub = ubs.pop() if ubs else 0.0
        f32 = np.empty(max(d, h), dtype=np.float32)
        codes = np.empty(max(d, h), dtype=np.uint8)
    elif bf16:
        w1, k1 = arr("w1", np.uint16); w3, k2 = arr("w3", np.uint16)
        w2, k3 = arr("w2", np.uint16)
        keep = (k1, k2, k3)  # noqa: F841  (keeps arrays alive)
    else:
        c1, k1 = arr("c1", np.int8); s1, k2 = arr("s1", np.float32)
        c3, k3 = arr("c3", np.int8); s3, k4 = arr("s3", np.float32)
        c2, k5 = arr("c2", np.int8); s2, k6 = arr("s2", np.float32)
        keep = (k1, k2, k3, k4, k5, k6)  # noqa: F841  (keeps arrays alive)

    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, top_k), dtype=np.int32)
    gates = np.empty((T, top_k), dtype=np.float64)
    y = np.empty((T, d), dtype=np.float64)
    u = np.empty(h, dtype=np.float64)
    o = np.empty(d, dtype=np.float64)
    forced = None if forced_ids is None else np.ascontiguousarray(forced_ids, dtype=np.int32)
    L = lib()
    for t in range(T):
        tail = (_ptr(sh1), _ptr(sh3), _ptr(sh2), None if forced is None else _ptr(forced[t]),
                _ptr(logits[t]), _ptr(ids[t]), _ptr(gates[t]), _ptr(u), _ptr(o), _ptr(y[t]))
        if fp8:
            rc = L.oracle_moe_token_fp8(_ptr(xf[t]), d, h, E, top_k, _ptr(wr),
                                        None if bias is None else _ptr(bias),
                                        q1, s1, q3, s3, q2, s2, ub, *tail[:7], _ptr(f32),
                                        _ptr(codes), *tail[7:])
        elif bf16:
            rc = L.oracle_moe_token_bf16(_ptr(xf[t]), d, h, E, top_k, _ptr(wr),
                                         None if bias is None else _ptr(bias), w1, w3, w2, *tail)
        else:
            rc = L.oracle_moe_token(_ptr(xf[t]), d, h, E, top_k, group_size, _ptr(wr),
                                    None if bias is None else _ptr(bias),
                                    c1, s1, c3, s3, c2, s2, *tail)
        if rc != 0:
            raise ValueError(f"token {t}: a chosen expert's weights were not supplied")
    if top_k < E:
        srt = -np.sort(-logits, axis=1)
        margin = (srt[:, top_k - 1].astype(np.float64) - srt[:, top_k]).astype(np.float32)
    else:
        margin = np.full(T, np.inf, dtype=np.float32)
    return MoEResult(y=y, ids=ids, gates=gates, logits=logits, margin=margin)

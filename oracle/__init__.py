"""Python access to the float64 CPU oracle of the fused MoE + multi-LoRA layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the library. It shares no code with the HIP path and does not
import it. The arithmetic lives in moelora_oracle.c; this file only marshals arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moelora_oracle.c")
_LIB = os.path.join(_HERE, "libmoelora_oracle.so")

ORC_BF16, ORC_F32, ORC_F64, ORC_FP8E4M3 = 0, 1, 2, 3


def build() -> str:
    """Compile the oracle with gcc (host code only)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", _SRC, "-o", _LIB, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "hidden", "inter", "n_experts", "n_adapters", "rank", "topk")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        L.oracle_route.argtypes = [P, i32, i32, i32, P, P]
        L.oracle_align.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, ctypes.c_int64, P, P, i32, P]
        L.oracle_forward.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, i32, P, P]
        L.oracle_forward_scaled.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, i32, P, P]
        L.oracle_fp8e4m3_decode.argtypes = [P, ctypes.c_int64, P]
        L.oracle_sgmv.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, P]
        L.oracle_router_logits.argtypes = [P, P, P, i32, i32, i32, P]
        L.oracle_num_threads.argtypes = []
        for f in (L.oracle_route, L.oracle_align, L.oracle_forward, L.oracle_forward_scaled,
                  L.oracle_fp8e4m3_decode, L.oracle_sgmv, L.oracle_router_logits,
                  L.oracle_num_threads):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _np(a):
    """numpy view of a CPU array or torch tensor; bf16 comes back as uint16 bit patterns, E4M3
    weight codes are uint8."""
    if hasattr(a, "detach"):
        import torch
        a = a.detach()
        if a.device.type != "cpu":
            raise ValueError("the oracle takes host arrays")
        if a.dtype == torch.bfloat16:
            return np.ascontiguousarray(a.contiguous().view(torch.int16).numpy().view(np.uint16)), ORC_BF16
        a = a.contiguous().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, ORC_BF16
    if a.dtype == np.uint8:
        return a, ORC_FP8E4M3
    if a.dtype == np.float32:
        return a, ORC_F32
    if a.dtype == np.float64:
        return a, ORC_F64
    raise TypeError(f"unsupported dtype {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def route(logits, k: int):
    """Top-k expert ids per token (slot order) and their softmax weights (float64)."""
    L, dtc = _np(logits)
    if dtc != ORC_F32:
        raise TypeError("router logits are float32")
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().oracle_route(_ptr(L), T, E, k, _ptr(ids), _ptr(w)), "oracle_route")
    return ids, w


def align(topk_ids, adapter_ids, n_experts: int, n_adapters: int, seg_pad: int = 1, block_m: int = 1):
    """Sorted pair list, padded expert offsets and segment table (see moelora_oracle.c)."""
    ids = _i32(topk_ids)
    ad = _i32(adapter_ids)
    T, k = ids.shape
    P = T * k
    cap = P * seg_pad + n_experts * block_m
    sp = np.empty(max(cap, 1), np.int32)
    off = np.empty(n_experts + 1, np.int32)
    seg_cap = max(P, 1)
    seg = np.empty((seg_cap, 4), np.int32)
    ns = np.zeros(1, np.int32)
    _check(lib().oracle_align(_ptr(ids), _ptr(ad), T, k, n_experts, n_adapters, seg_pad, block_m,
                              _ptr(sp), cap, _ptr(off), _ptr(seg), seg_cap, _ptr(ns)), "oracle_align")
    total = int(off[-1])
    return {"sorted_pairs": sp[:total].copy(), "expert_offsets": off, "seg_table": seg[: int(ns[0])].copy(),
            "n_seg": int(ns[0])}


def forward(inputs: dict, topk: int, tokens=None, return_pairs: bool = False):
    """y[len(tokens)][h] in float64 (all tokens when tokens is None).

    `inputs` holds x, logits, W1, W2, A1, B1, A2, B2, adapter_ids with the stored layouts
    x[T][h], W1[E][2I][h], W2[E][h][I], A1[nA][E][r][h], B1[nA][E][2I][r], A2[nA][E][r][I],
    B2[nA][E][h][r]; each may be bf16, float32 or float64. W1 and W2 may instead be uint8 E4M3
    codes, with their per-row scales in inputs["W1_scale"] [E][2I] and inputs["W2_scale"]
    [E][h] (float32)."""
    arrs = []
    dts = []
    for name in ("x", "W1", "W2", "A1", "B1", "A2", "B2"):
        a, dtc = _np(inputs[name])
        arrs.append(a)
        dts.append(dtc)
    x, W1, W2, A1, B1, A2, B2 = arrs
    T, h = x.shape
    E, twoI, h1 = W1.shape
    I = twoI // 2
    nA, E1, r, h2 = A1.shape
    if not (h1 == h2 == h and E1 == E and W2.shape == (E, h, I) and B1.shape == (nA, E, 2 * I, r)
            and A2.shape == (nA, E, r, I) and B2.shape == (nA, E, h, r)):
        raise ValueError("inconsistent shapes")
    L, ldt = _np(inputs["logits"])
    if ldt != ORC_F32 or L.shape != (T, E):
        raise ValueError("logits must be float32 [T][E]")
    ad = _i32(inputs["adapter_ids"])
    if ad.shape != (T,):
        raise ValueError("adapter_ids must be [T]")
    dims = _Dims(T, h, I, E, nA, r, topk)
    if tokens is None:
        toks = None
        n = T
    else:
        toks = _i32(tokens).reshape(-1)
        n = toks.size
    y = np.zeros((n, h), np.float64)
    dp = np.zeros((n, topk, h), np.float64) if return_pairs else None
    tptr = (ctypes.c_void_p * 7)(*[a.ctypes.data for a in arrs])
    dtarr = (ctypes.c_int32 * 7)(*dts)
    scales = []
    for name, shape in (("W1_scale", (E, 2 * I)), ("W2_scale", (E, h))):
        sc = inputs.get(name)
        if sc is None:
            scales.append(None)
            continue
        sc, sdt = _np(sc)
        if sdt != ORC_F32 or sc.shape != shape:
            raise ValueError(f"{name} must be float32 {shape}")
        scales.append(sc)
    rc = lib().oracle_forward_scaled(ctypes.byref(dims), tptr, dtarr,
                                     None if scales[0] is None else _ptr(scales[0]),
                                     None if scales[1] is None else _ptr(scales[1]), _ptr(L),
                                     _ptr(ad), None if toks is None else _ptr(toks), n, _ptr(y),
                                     None if dp is None else _ptr(dp))
    _check(rc, "oracle_forward")
    return (y, dp) if return_pairs else y


def router_logits(x, W_router) -> np.ndarray:
    """logits[T][E] = x W_router^T in float64 (x [T][h], W_router [E][h]; bf16, f32 or f64)."""
    xa, dx = _np(x)
    wa, dw = _np(W_router)
    T, h = xa.shape
    E, h2 = wa.shape
    if h2 != h or ORC_FP8E4M3 in (dx, dw):
        raise ValueError("x [T][h] and W_router [E][h] (bf16, f32 or f64)")
    out = np.zeros((T, E), np.float64)
    dtarr = (ctypes.c_int32 * 2)(dx, dw)
    _check(lib().oracle_router_logits(_ptr(xa), _ptr(wa), dtarr, T, h, E, _ptr(out)), "oracle_router_logits")
    return out


def sgmv(x, A, B, y_in, adapter_ids) -> np.ndarray:
    """Dense multi-LoRA: y_in + (x A_a^T) B_a^T per token (a = adapter_ids[t], -1: unchanged),
    float64. x[T][K], A[nA][r][K], B[nA][N][r], y_in[T][N]; bf16, float32 or float64 each."""
    arrs, dts = [], []
    for a in (x, A, B, y_in):
        v, dtc = _np(a)
        if dtc == ORC_FP8E4M3:
            raise TypeError("E4M3 is for the expert weights only")
        arrs.append(v)
        dts.append(dtc)
    xa, Aa, Ba, ya = arrs
    T, K = xa.shape
    nA, r, K2 = Aa.shape
    nA2, N, r2 = Ba.shape
    if K2 != K or nA2 != nA or r2 != r or ya.shape != (T, N):
        raise ValueError("inconsistent shapes")
    ad = _i32(adapter_ids)
    if ad.shape != (T,):
        raise ValueError("adapter_ids must be [T]")
    out = np.zeros((T, N), np.float64)
    dtarr = (ctypes.c_int32 * 4)(*dts)
    _check(lib().oracle_sgmv(_ptr(xa), _ptr(Aa), _ptr(Ba), _ptr(ya), dtarr, _ptr(ad), T, K, N, nA, r,
                             _ptr(out)), "oracle_sgmv")
    return out


def fp8e4m3_decode(codes) -> np.ndarray:
    """float64 values of uint8 E4M3 codes (any shape)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    _check(lib().oracle_fp8e4m3_decode(_ptr(c), c.size, _ptr(out)), "oracle_fp8e4m3_decode")
    return out


def num_threads() -> int:
    return int(lib().oracle_num_threads())

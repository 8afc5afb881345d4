"""Fused MoE + multi-LoRA layer for AMD Instinct MI355X (gfx950).

Thin ctypes binding over libmoelora.so (include/moelora.h). Every step of the layer runs in
the library's HIP kernels; this module only checks tensor shapes, allocates outputs and the
workspace with torch when the caller does not pass them, and hands raw device pointers and
torch's current HIP stream to the C ABI. There is no fallback: without the built library or
a gfx950 device every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoelora.so")

OK, EINVAL_DIMS, ENULL, EALIGN, EWORKSPACE, EHIP, EDEVICE, EUNSUPPORTED, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8
FLAG_NONFINITE_LOGIT, FLAG_ADAPTER_RANGE = 1, 2

EXPORTS = ("moe_lora_workspace_size", "moe_lora_forward", "moe_lora_forward_timed", "moe_lora_forward_fp8",
           "moe_lora_sorted_capacity", "moe_lora_route_align", "moe_lora_strerror",
           "moe_lora_debug_status", "moe_lora_sgmv_workspace_size", "moe_lora_sgmv",
           "moe_lora_router_logits", "moe_lora_forward_routed", "moe_lora_workspace_layout",
           "moe_lora_forward_noalloc", "moe_lora_probe_read", "moe_lora_probe_mfma")
N_STAGES = 7
STAGES = ("route", "align", "shrink_gate_up", "gate_up", "shrink_down", "down", "combine")


class MoeLoraError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (code {code})")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "hidden", "inter", "n_experts", "n_adapters", "rank")]


class LayoutInfo(ctypes.Structure):
    _fields_ = [("tiled", ctypes.c_int32), ("block_m", ctypes.c_int32)] + [
        (n, ctypes.c_int64) for n in ("capacity", "workspace_bytes", "topk_ids", "topk_w", "sorted_pairs",
                                      "expert_offsets", "seg_table", "n_seg", "n_blocks", "block_expert",
                                      "block_seg", "pair_row", "sorted_ad")]


class SgmvDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "in_features", "out_features", "n_adapters", "rank")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with lora_mixture_experts_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        D = ctypes.POINTER(Dims)
        L.moe_lora_workspace_size.argtypes = [D, i32]
        L.moe_lora_workspace_size.restype = ctypes.c_size_t
        L.moe_lora_forward.argtypes = [P, P, P, P, P, P, P, P, P, i32, D, P, P, ctypes.c_size_t, P]
        L.moe_lora_forward.restype = ctypes.c_int
        L.moe_lora_forward_timed.argtypes = [P, P, P, P, P, P, P, P, P, i32, D, P, P, ctypes.c_size_t, P,
                                             ctypes.POINTER(ctypes.c_void_p)]
        L.moe_lora_forward_timed.restype = ctypes.c_int
        L.moe_lora_forward_fp8.argtypes = [P, P, P, P, P, P, P, P, P, P, P, i32, D, P, P, ctypes.c_size_t, P,
                                           ctypes.POINTER(ctypes.c_void_p)]
        L.moe_lora_forward_fp8.restype = ctypes.c_int
        L.moe_lora_probe_read.argtypes = [P, ctypes.c_size_t, P, P]
        L.moe_lora_probe_read.restype = ctypes.c_int
        L.moe_lora_probe_mfma.argtypes = [i32, i32, P, P]
        L.moe_lora_probe_mfma.restype = ctypes.c_int
        L.moe_lora_forward_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, i32, D, P, P]
        L.moe_lora_forward_noalloc.restype = ctypes.c_int
        L.moe_lora_router_logits.argtypes = [P, P, i32, i32, i32, P, P]
        L.moe_lora_router_logits.restype = ctypes.c_int
        L.moe_lora_forward_routed.argtypes = [P, P, P, P, P, P, P, P, P, i32, D, P, P, ctypes.c_size_t, P]
        L.moe_lora_forward_routed.restype = ctypes.c_int
        L.moe_lora_sgmv_workspace_size.argtypes = [ctypes.POINTER(SgmvDims)]
        L.moe_lora_sgmv_workspace_size.restype = ctypes.c_size_t
        L.moe_lora_sgmv.argtypes = [P, P, P, P, ctypes.POINTER(SgmvDims), P, P, ctypes.c_size_t, P]
        L.moe_lora_sgmv.restype = ctypes.c_int
        L.moe_lora_sorted_capacity.argtypes = [D, i32, i32, i32]
        L.moe_lora_sorted_capacity.restype = i64
        L.moe_lora_route_align.argtypes = [P, P, i32, D, i32, i32, P, P, P, i64, P, P, P, P,
                                           ctypes.c_size_t, P]
        L.moe_lora_route_align.restype = ctypes.c_int
        L.moe_lora_workspace_layout.argtypes = [D, i32, ctypes.POINTER(LayoutInfo)]
        L.moe_lora_workspace_layout.restype = ctypes.c_int
        L.moe_lora_strerror.argtypes = [ctypes.c_int]
        L.moe_lora_strerror.restype = ctypes.c_char_p
        L.moe_lora_debug_status.argtypes = [P, ctypes.c_size_t, P, ctypes.POINTER(ctypes.c_uint32)]
        L.moe_lora_debug_status.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_lora_strerror(code).decode()


def _check(code: int, what: str):
    if code != OK:
        raise MoeLoraError(code, what)


def dims_of(x: torch.Tensor, W1: torch.Tensor, A1: torch.Tensor) -> Dims:
    T, h = x.shape
    E, twoI, _ = W1.shape
    nA, _, r, _ = A1.shape
    return Dims(T, h, twoI // 2, E, nA, r)


def workspace_size(d: Dims, topk: int) -> int:
    return int(lib().moe_lora_workspace_size(ctypes.byref(d), topk))


def sorted_capacity(d: Dims, topk: int, seg_pad: int, block_m: int) -> int:
    return int(lib().moe_lora_sorted_capacity(ctypes.byref(d), topk, seg_pad, block_m))


def new_workspace(d: Dims, topk: int, device) -> torch.Tensor:
    n = workspace_size(d, topk)
    if n == 0:
        raise MoeLoraError(EINVAL_DIMS, "workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def workspace_layout(d: Dims, topk: int) -> dict:
    """Where the forward keeps its sorted layout in the workspace (moe_lora_workspace_layout)."""
    info = LayoutInfo()
    _check(lib().moe_lora_workspace_layout(ctypes.byref(d), topk, ctypes.byref(info)),
           "moe_lora_workspace_layout")
    return {name: getattr(info, name) for name, _ in LayoutInfo._fields_}


def read_layout_tables(workspace: torch.Tensor, d: Dims, topk: int) -> dict:
    """The forward's routing and sorted-layout tables, copied to the host from the workspace of
    the last call that used it (int32 numpy arrays; topk_w float32). Synchronises."""
    info = workspace_layout(d, topk)
    host = workspace.cpu()
    P = d.T * topk

    def region(name, n, dtype=torch.int32):
        off = info[name]
        return host[off:off + 4 * n].view(dtype).numpy()

    n_blocks = int(region("n_blocks", 1)[0])
    n_seg = int(region("n_seg", 1)[0])
    total = n_blocks * info["block_m"]
    return {
        "info": info, "n_blocks": n_blocks, "n_seg": n_seg,
        "topk_ids": region("topk_ids", P).reshape(d.T, topk),
        "topk_w": region("topk_w", P, torch.float32).reshape(d.T, topk),
        "sorted_pairs": region("sorted_pairs", total),
        "expert_offsets": region("expert_offsets", d.n_experts + 1),
        "seg_table": region("seg_table", 4 * n_seg).reshape(n_seg, 4),
        "block_expert": region("block_expert", n_blocks),
        "block_seg": region("block_seg", n_blocks),
        "pair_row": region("pair_row", P),
        "sorted_ad": region("sorted_ad", total),
    }


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _expect(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")


def forward(x, router_logits, W1, W2, A1, B1, A2, B2, adapter_ids, topk: int, y=None,
            workspace=None, stage_events=None) -> torch.Tensor:
    """y[T][h] (bf16) of the fused MoE + multi-LoRA layer; see include/moelora.h.

    stage_events: optional list of N_STAGES + 1 torch.cuda.Event(enable_timing=True) (or None
    for a boundary not to record) that the library records at the stage boundaries on the
    current stream (moe_lora_forward_timed)."""
    d = dims_of(x, W1, A1)
    T, h, I, E, nA, r = d.T, d.hidden, d.inter, d.n_experts, d.n_adapters, d.rank
    bf = torch.bfloat16
    _expect(x, "x", bf, (T, h))
    _expect(router_logits, "router_logits", torch.float32, (T, E))
    _expect(W1, "W1", bf, (E, 2 * I, h))
    _expect(W2, "W2", bf, (E, h, I))
    _expect(A1, "A1", bf, (nA, E, r, h))
    _expect(B1, "B1", bf, (nA, E, 2 * I, r))
    _expect(A2, "A2", bf, (nA, E, r, I))
    _expect(B2, "B2", bf, (nA, E, h, r))
    _expect(adapter_ids, "adapter_ids", torch.int32, (T,))
    if y is None:
        y = torch.empty((T, h), dtype=bf, device=x.device)
    _expect(y, "y", bf, (T, h))
    if workspace is None:
        workspace = new_workspace(d, topk, x.device)
    args = (_ptr(x), _ptr(router_logits), _ptr(W1), _ptr(W2), _ptr(A1), _ptr(B1), _ptr(A2), _ptr(B2),
            _ptr(adapter_ids), topk, ctypes.byref(d), _ptr(y), _ptr(workspace), workspace.numel(),
            _stream(x.device))
    if stage_events is None:
        _check(lib().moe_lora_forward(*args), "moe_lora_forward")
    else:
        if len(stage_events) != N_STAGES + 1:
            raise ValueError(f"need {N_STAGES + 1} events")
        for ev in stage_events:
            if ev is not None and not ev.cuda_event:  # torch creates the HIP event on its first record
                ev.record()
        handles = (ctypes.c_void_p * (N_STAGES + 1))(
            *[ev.cuda_event if ev is not None else None for ev in stage_events])
        _check(lib().moe_lora_forward_timed(*args, handles), "moe_lora_forward_timed")
    return y


def forward_noalloc(x, router_logits, W1, W2, A1, B1, A2, B2, adapter_ids, topk: int,
                    y=None) -> torch.Tensor:
    """forward without a workspace argument (moe_lora_forward_noalloc): the library uses its
    static 128 MiB device scratch. Raises MoeLoraError(ESCRATCH) when the sizes need more.
    Calls on one GPU share that scratch and must be ordered on one stream."""
    d = dims_of(x, W1, A1)
    T, h, I, E, nA, r = d.T, d.hidden, d.inter, d.n_experts, d.n_adapters, d.rank
    bf = torch.bfloat16
    _expect(x, "x", bf, (T, h))
    _expect(router_logits, "router_logits", torch.float32, (T, E))
    _expect(W1, "W1", bf, (E, 2 * I, h))
    _expect(W2, "W2", bf, (E, h, I))
    _expect(A1, "A1", bf, (nA, E, r, h))
    _expect(B1, "B1", bf, (nA, E, 2 * I, r))
    _expect(A2, "A2", bf, (nA, E, r, I))
    _expect(B2, "B2", bf, (nA, E, h, r))
    _expect(adapter_ids, "adapter_ids", torch.int32, (T,))
    if y is None:
        y = torch.empty((T, h), dtype=bf, device=x.device)
    _expect(y, "y", bf, (T, h))
    _check(lib().moe_lora_forward_noalloc(_ptr(x), _ptr(router_logits), _ptr(W1), _ptr(W2), _ptr(A1),
                                          _ptr(B1), _ptr(A2), _ptr(B2), _ptr(adapter_ids), topk,
                                          ctypes.byref(d), _ptr(y), _stream(x.device)),
           "moe_lora_forward_noalloc")
    return y


def router_logits(x, W_router, out=None) -> torch.Tensor:
    """logits [T][E] float32 = x W_router^T (moe_lora_router_logits), into `out` if given."""
    T, h = x.shape
    E = W_router.shape[0]
    _expect(x, "x", torch.bfloat16, (T, h))
    _expect(W_router, "W_router", torch.bfloat16, (E, h))
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _expect(out, "out", torch.float32, (T, E))
    _check(lib().moe_lora_router_logits(_ptr(x), _ptr(W_router), T, h, E, _ptr(out), _stream(x.device)),
           "moe_lora_router_logits")
    return out


def forward_routed(x, W_router, W1, W2, A1, B1, A2, B2, adapter_ids, topk: int, y=None,
                   workspace=None) -> torch.Tensor:
    """forward starting from the router weights W_router [E][h] (moe_lora_forward_routed)."""
    d = dims_of(x, W1, A1)
    T, h, I, E, nA, r = d.T, d.hidden, d.inter, d.n_experts, d.n_adapters, d.rank
    bf = torch.bfloat16
    _expect(x, "x", bf, (T, h))
    _expect(W_router, "W_router", bf, (E, h))
    _expect(W1, "W1", bf, (E, 2 * I, h))
    _expect(W2, "W2", bf, (E, h, I))
    _expect(A1, "A1", bf, (nA, E, r, h))
    _expect(B1, "B1", bf, (nA, E, 2 * I, r))
    _expect(A2, "A2", bf, (nA, E, r, I))
    _expect(B2, "B2", bf, (nA, E, h, r))
    _expect(adapter_ids, "adapter_ids", torch.int32, (T,))
    if y is None:
        y = torch.empty((T, h), dtype=bf, device=x.device)
    _expect(y, "y", bf, (T, h))
    if workspace is None:
        workspace = new_workspace(d, topk, x.device)
    _check(lib().moe_lora_forward_routed(_ptr(x), _ptr(W_router), _ptr(W1), _ptr(W2), _ptr(A1), _ptr(B1),
                                         _ptr(A2), _ptr(B2), _ptr(adapter_ids), topk, ctypes.byref(d),
                                         _ptr(y), _ptr(workspace), workspace.numel(), _stream(x.device)),
           "moe_lora_forward_routed")
    return y


def sgmv(x, A, B, adapter_ids, y, workspace=None) -> torch.Tensor:
    """Dense multi-LoRA, in place: y[t] += (x[t] A[a]^T) B[a]^T for a = adapter_ids[t] (-1: y[t]
    unchanged); moe_lora_sgmv. x [T][K], A [nA][r][K], B [nA][N][r], y [T][N] bf16,
    adapter_ids [T] int32."""
    T, K = x.shape
    nA, r, _ = A.shape
    N = B.shape[1]
    d = SgmvDims(T, K, N, nA, r)
    bf = torch.bfloat16
    _expect(x, "x", bf, (T, K))
    _expect(A, "A", bf, (nA, r, K))
    _expect(B, "B", bf, (nA, N, r))
    _expect(adapter_ids, "adapter_ids", torch.int32, (T,))
    _expect(y, "y", bf, (T, N))
    if workspace is None:
        n = int(lib().moe_lora_sgmv_workspace_size(ctypes.byref(d)))
        if n == 0:
            raise MoeLoraError(EINVAL_DIMS, "moe_lora_sgmv_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    _check(lib().moe_lora_sgmv(_ptr(x), _ptr(A), _ptr(B), _ptr(adapter_ids), ctypes.byref(d), _ptr(y),
                               _ptr(workspace), workspace.numel(), _stream(x.device)), "moe_lora_sgmv")
    return y


def forward_fp8(x, router_logits, W1q, W1_scale, W2q, W2_scale, A1, B1, A2, B2, adapter_ids,
                topk: int, y=None, workspace=None, stage_events=None) -> torch.Tensor:
    """forward with E4M3 expert weights (moe_lora_forward_fp8): W1q [E][2I][h] and W2q [E][h][I]
    as uint8 codes, W1_scale [E][2I] and W2_scale [E][h] float32 per-row scales; the rest as
    in forward."""
    T, h = x.shape
    E, twoI, _ = W1q.shape
    nA, _, r, _ = A1.shape
    I = twoI // 2
    d = Dims(T, h, I, E, nA, r)
    bf = torch.bfloat16
    _expect(x, "x", bf, (T, h))
    _expect(router_logits, "router_logits", torch.float32, (T, E))
    _expect(W1q, "W1q", torch.uint8, (E, 2 * I, h))
    _expect(W1_scale, "W1_scale", torch.float32, (E, 2 * I))
    _expect(W2q, "W2q", torch.uint8, (E, h, I))
    _expect(W2_scale, "W2_scale", torch.float32, (E, h))
    _expect(A1, "A1", bf, (nA, E, r, h))
    _expect(B1, "B1", bf, (nA, E, 2 * I, r))
    _expect(A2, "A2", bf, (nA, E, r, I))
    _expect(B2, "B2", bf, (nA, E, h, r))
    _expect(adapter_ids, "adapter_ids", torch.int32, (T,))
    if y is None:
        y = torch.empty((T, h), dtype=bf, device=x.device)
    _expect(y, "y", bf, (T, h))
    if workspace is None:
        workspace = new_workspace(d, topk, x.device)
    handles = None
    if stage_events is not None:
        if len(stage_events) != N_STAGES + 1:
            raise ValueError(f"need {N_STAGES + 1} events")
        for ev in stage_events:
            if ev is not None and not ev.cuda_event:
                ev.record()
        handles = (ctypes.c_void_p * (N_STAGES + 1))(
            *[ev.cuda_event if ev is not None else None for ev in stage_events])
    _check(lib().moe_lora_forward_fp8(_ptr(x), _ptr(router_logits), _ptr(W1q), _ptr(W1_scale),
                                      _ptr(W2q), _ptr(W2_scale), _ptr(A1), _ptr(B1), _ptr(A2),
                                      _ptr(B2), _ptr(adapter_ids), topk, ctypes.byref(d), _ptr(y),
                                      _ptr(workspace), workspace.numel(), _stream(x.device), handles),
           "moe_lora_forward_fp8")
    return y


def route_align(router_logits, adapter_ids, topk: int, d: Dims, seg_pad: int = 1, block_m: int = 1,
                workspace=None) -> dict:
    """Routing and align outputs as device tensors; see moe_lora_route_align."""
    dev = router_logits.device
    _expect(router_logits, "router_logits", torch.float32, (d.T, d.n_experts))
    _expect(adapter_ids, "adapter_ids", torch.int32, (d.T,))
    cap = sorted_capacity(d, topk, seg_pad, block_m)
    if cap < 0:
        raise MoeLoraError(EINVAL_DIMS, "sorted_capacity")
    P = d.T * topk
    out = {
        "topk_ids": torch.empty((d.T, topk), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((d.T, topk), dtype=torch.float32, device=dev),
        "sorted_pairs": torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev),
        "expert_offsets": torch.empty(d.n_experts + 1, dtype=torch.int32, device=dev),
        "seg_table": torch.empty((max(P, 1), 4), dtype=torch.int32, device=dev),
        "n_seg": torch.empty(1, dtype=torch.int32, device=dev),
    }
    if workspace is None:
        workspace = new_workspace(d, topk, dev)
    rc = lib().moe_lora_route_align(_ptr(router_logits), _ptr(adapter_ids), topk, ctypes.byref(d),
                                    seg_pad, block_m, _ptr(out["topk_ids"]), _ptr(out["topk_w"]),
                                    _ptr(out["sorted_pairs"]), cap, _ptr(out["expert_offsets"]),
                                    _ptr(out["seg_table"]), _ptr(out["n_seg"]), _ptr(workspace),
                                    workspace.numel(), _stream(dev))
    _check(rc, "moe_lora_route_align")
    out["workspace"] = workspace
    return out


PROBE_READ_SINK = 2048 * 256  # uint32 words the read probe writes


def probe_read(src: torch.Tensor, sink: torch.Tensor):
    """Streaming read of src's bytes (moe_lora_probe_read) on the current stream."""
    _check(lib().moe_lora_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                     _stream(src.device)), "moe_lora_probe_read")


def probe_mfma(iters: int, n_workgroups: int, sink: torch.Tensor) -> int:
    """Loop of bf16 MFMAs (moe_lora_probe_mfma) on the current stream; returns its flops."""
    _check(lib().moe_lora_probe_mfma(iters, n_workgroups, _ptr(sink), _stream(sink.device)),
           "moe_lora_probe_mfma")
    return n_workgroups * 4 * iters * 8 * 32768


def debug_status(workspace: torch.Tensor) -> int:
    """Device flags (FLAG_* bits) of the last call that used `workspace`; synchronises."""
    flags = ctypes.c_uint32(0)
    rc = lib().moe_lora_debug_status(_ptr(workspace), workspace.numel(), _stream(workspace.device),
                                     ctypes.byref(flags))
    _check(rc, "moe_lora_debug_status")
    return int(flags.value)

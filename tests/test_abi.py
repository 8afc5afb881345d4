"""The C ABI library loads on a host without a GPU, exports every entry point the header
declares, and rejects bad arguments on the host before any device call. CPU only."""
import ctypes
import os
import re

import pytest

import lora_mixture_experts_amd as ml
from lora_mixture_experts_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_lora_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = ml.lib()
    declared = _declared()
    assert declared == set(ml.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_workspace_size_and_capacity():
    d = Dims(64, 4096, 11008, 16, 8, 16)
    n = ml.workspace_size(d, 2)
    assert n > 2 * 128 * 11008 * 2  # at least the intermediate activations
    assert n % 256 == 0
    assert ml.sorted_capacity(d, 2, 1, 16) == 128 + 16 * 15
    assert ml.sorted_capacity(d, 2, 4, 64) == 128 * 4 + 16 * 63
    assert ml.sorted_capacity(d, 2, 0, 16) == -1
    assert ml.sorted_capacity(d, 2, 1, 257) == -1


@pytest.mark.parametrize("bad", [
    dict(hidden=100), dict(inter=64 * 3), dict(rank=12), dict(n_experts=0), dict(n_experts=2000),
    dict(n_adapters=0), dict(T=-1), dict(hidden=0),
])
def test_workspace_size_rejects_bad_dims(bad):
    base = dict(T=16, hidden=256, inter=512, n_experts=8, n_adapters=4, rank=8)
    base.update(bad)
    assert ml.workspace_size(Dims(**base), 2) == 0


@pytest.mark.parametrize("topk", [0, 9, 17])
def test_workspace_size_rejects_bad_topk(topk):
    assert ml.workspace_size(Dims(16, 256, 512, 8, 4, 8), topk) == 0


def test_strerror_covers_codes():
    for code in (ml.OK, ml.EINVAL_DIMS, ml.ENULL, ml.EALIGN, ml.EWORKSPACE, ml.EHIP, ml.EDEVICE):
        assert ml.strerror(code) not in ("", "unknown error code")
    assert ml.strerror(123) == "unknown error code"


def _fwd(ptrs, d, topk=2, ws_bytes=None):
    lib = ml.lib()
    if ws_bytes is None:
        ws_bytes = ml.workspace_size(d, topk) if ml.workspace_size(d, topk) else 1 << 40
    return lib.moe_lora_forward(*ptrs[:9], topk, ctypes.byref(d), ptrs[9], ptrs[10], ws_bytes, None)


FAKE = [0x10000 * (i + 1) for i in range(11)]  # aligned, never dereferenced: checks fail first


def test_forward_host_validation_without_device():
    d = Dims(16, 256, 512, 8, 4, 8)
    for i in range(11):
        p = list(FAKE)
        p[i] = None
        assert _fwd(p, d) == ml.ENULL
    for i in range(10):
        p = list(FAKE)
        p[i] += 8
        assert _fwd(p, d) == ml.EALIGN
    p = list(FAKE)
    p[10] += 16  # workspace 16- but not 256-aligned
    assert _fwd(p, d) == ml.EWORKSPACE
    assert _fwd(FAKE, d, ws_bytes=ml.workspace_size(d, 2) - 1) == ml.EWORKSPACE
    assert _fwd(FAKE, Dims(16, 250, 512, 8, 4, 8)) == ml.EINVAL_DIMS
    assert _fwd(FAKE, d, topk=9) == ml.EINVAL_DIMS
    # T = 0 is a valid empty call: nothing is enqueued, no pointer is read, no device is needed
    assert _fwd(FAKE, Dims(0, 256, 512, 8, 4, 8)) == ml.OK
    assert _fwd([None] * 11, Dims(0, 256, 512, 8, 4, 8)) == ml.OK


def test_route_align_host_validation_without_device():
    lib = ml.lib()
    d = Dims(16, 256, 512, 8, 4, 8)
    ws = ml.workspace_size(d, 2)
    cap = ml.sorted_capacity(d, 2, 1, 16)
    p = [0x10000 * (i + 1) for i in range(9)]

    def call(pp, cap_=cap, seg_pad=1, block_m=16, ws_=ws):
        return lib.moe_lora_route_align(pp[0], pp[1], 2, ctypes.byref(d), seg_pad, block_m, pp[2], pp[3],
                                        pp[4], cap_, pp[5], pp[6], pp[7], pp[8], ws_, None)

    assert call(p, cap_=cap - 1) == ml.EINVAL_DIMS
    assert call(p, seg_pad=0) == ml.EINVAL_DIMS
    for i in range(9):
        q = list(p)
        q[i] = None
        assert call(q) == ml.ENULL
    q = list(p)
    q[2] += 2
    assert call(q) == ml.EALIGN
    assert call(p, ws_=ws - 1) == ml.EWORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        ml._expect(x, "x", torch.bfloat16, (4, 128))


def _routed(ptrs, d, topk=2, ws_bytes=None):
    """moe_lora_forward_routed with ptrs = x, W_router, W1, W2, A1, B1, A2, B2, adapter_ids, y,
    workspace (aligned fake addresses that the host checks reject before any device call)."""
    if ws_bytes is None:
        ws_bytes = ml.workspace_size(d, topk) if ml.workspace_size(d, topk) else 1 << 40
    return ml.lib().moe_lora_forward_routed(*ptrs[:9], topk, ctypes.byref(d), ptrs[9], ptrs[10],
                                            ws_bytes, None)


def test_forward_routed_host_validation_without_device():
    """Every pointer of the routed entry (W1 included) is checked before the router GEMM is
    enqueued: with no GPU here, any enqueue would fail with EHIP or EDEVICE instead."""
    d = Dims(16, 256, 512, 8, 4, 8)
    for i in range(11):
        p = list(FAKE)
        p[i] = None
        assert _routed(p, d) == ml.ENULL, i
    for i in range(10):
        p = list(FAKE)
        p[i] += 8
        assert _routed(p, d) == ml.EALIGN, i
    p = list(FAKE)
    p[10] += 16
    assert _routed(p, d) == ml.EWORKSPACE
    assert _routed(FAKE, d, ws_bytes=ml.workspace_size(d, 2) - 1) == ml.EWORKSPACE
    assert _routed(FAKE, Dims(16, 250, 512, 8, 4, 8)) == ml.EINVAL_DIMS
    assert _routed([None] * 11, Dims(0, 256, 512, 8, 4, 8)) == ml.OK


def test_forward_fp8_host_validation_without_device():
    lib = ml.lib()
    d = Dims(16, 256, 512, 8, 4, 8)
    # x, logits, W1q, W1_scale, W2q, W2_scale, A1, B1, A2, B2, adapter_ids, y, workspace
    base = [0x10000 * (i + 1) for i in range(13)]

    def call(pp, dd=d, topk=2):
        return lib.moe_lora_forward_fp8(*pp[:11], topk, ctypes.byref(dd), pp[11], pp[12],
                                        ml.workspace_size(dd, topk), None, None)

    for i in range(13):
        q = list(base)
        q[i] = None
        assert call(q) == ml.ENULL, i
    q = list(base)
    q[3] += 2  # scales need 4-byte alignment
    assert call(q) == ml.EALIGN
    # above 24 token-expert pairs per expert (the LDS-tiled path) the FP8 entry is accepted too:
    # the host checks pass, and with no GPU here the device check fails
    big = Dims(200, 256, 512, 8, 4, 8)
    assert call(base, dd=big) in (ml.EHIP, ml.EDEVICE)


def test_workspace_layout_follows_the_path():
    """The workspace is sized for the path a call takes: weight-streaming calls (few rows per
    expert) reserve 16- or 32-row blocks, tiled calls 64 to 256; every region lies inside it."""
    decode = Dims(64, 4096, 11008, 16, 8, 16)
    info = ml.workspace_layout(decode, 2)
    assert info["tiled"] == 0 and info["block_m"] == 16
    assert info["capacity"] == 512  # 128 pairs + 16 experts x 15 padding rows, rounded to 256
    assert info["workspace_bytes"] == ml.workspace_size(decode, 2)
    assert info["workspace_bytes"] < 64 << 20
    prefill = Dims(4096, 4096, 14336, 8, 32, 64)
    info = ml.workspace_layout(prefill, 2)
    assert info["tiled"] == 1 and info["block_m"] == 256
    assert info["capacity"] == 8192 + 8 * 256
    regions = ("topk_ids", "topk_w", "sorted_pairs", "expert_offsets", "seg_table", "n_seg", "n_blocks",
               "block_expert", "block_seg", "pair_row", "sorted_ad")
    for dd in (decode, prefill, Dims(256, 2048, 768, 128, 64, 32), Dims(1024, 4096, 11008, 16, 1024, 16)):
        info = ml.workspace_layout(dd, 2 if dd.n_experts < 128 else 8)
        offs = sorted(info[r] for r in regions)
        assert len(set(offs)) == len(offs)
        assert all(o % 256 == 0 and 0 < o < info["workspace_bytes"] for o in offs)
    with pytest.raises(ml.MoeLoraError):
        ml.workspace_layout(Dims(16, 250, 512, 8, 4, 8), 2)


def test_activations_over_2gib_rejected():
    """The activations [capacity][inter] bf16 are read with 32-bit offsets: sizes whose
    capacity times inter reaches 2 GiB are refused, judged on the capacity the path uses."""
    # 128-row tiles: capacity = round_up(T*k + 127*E, 256)
    ok = Dims(200000, 128, 4096, 1, 1, 8)
    assert ml.workspace_size(ok, 1) > 0
    too_big = Dims(270000, 128, 4096, 1, 1, 8)  # 270 K rows x 4096 x 2 B > 2 GiB
    assert ml.workspace_size(too_big, 1) == 0


def test_forward_noalloc_host_validation_without_device():
    """The no-alloc entry takes no workspace: sizes whose workspace exceeds its 128 MiB scratch
    are refused with ESCRATCH, and pointers are checked, all before any device call."""
    lib = ml.lib()

    def call(ptrs, d, topk=2):
        return lib.moe_lora_forward_noalloc(*ptrs[:9], topk, ctypes.byref(d), ptrs[9], None)

    d = Dims(16, 256, 512, 8, 4, 8)
    for i in range(10):
        p = list(FAKE[:10])
        p[i] = None
        assert call(p, d) == ml.ENULL, i
        p = list(FAKE[:10])
        p[i] += 8
        assert call(p, d) == ml.EALIGN, i
    prefill = Dims(4096, 4096, 14336, 8, 32, 64)
    assert ml.workspace_size(prefill, 2) > 128 << 20
    assert call(FAKE[:10], prefill) == ml.ESCRATCH
    assert ml.strerror(ml.ESCRATCH) != "unknown error code"
    assert call([None] * 10, Dims(0, 256, 512, 8, 4, 8)) == ml.OK

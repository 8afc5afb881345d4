"""The entry point that allocates nothing (moe_lora_forward_noalloc): its static device scratch
stands in for the caller's workspace, and its output equals moe_lora_forward's, bit for bit and
within the oracle's bound, on two calls in a row, the second one smaller."""
import sys

import numpy as np
import pytest
import torch

import lora_mixture_experts_amd as ml
from synth import configs
from synth.configs import Workload
from tests.helpers import check_close, oracle_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pair(w: Workload, seed: int):
    inp = configs.make_inputs(w, seed, b_scale=10.0)
    inp["adapter_ids"][::5] = -1
    g = {k: v.to(DEV) for k, v in inp.items()}
    keys = ("x", "logits", "W1", "W2", "A1", "B1", "A2", "B2", "adapter_ids")
    y_ref = ml.forward(*[g[k] for k in keys], w.topk)
    y_na = ml.forward_noalloc(*[g[k] for k in keys], w.topk)
    torch.cuda.synchronize()
    return inp, y_ref, y_na


@pytest.mark.parametrize("big,small", [
    # weight-streaming path: a larger batch, then a smaller one (fewer rows in the scratch)
    (Workload("na_fg", 64, 256, 384, 32, 8, 16, 32, hot_experts=4, hot_bias=2.0),
     Workload("na_fg_small", 37, 256, 384, 32, 8, 16, 32, hot_experts=4, hot_bias=2.0)),
    # LDS-tiled path (64-row blocks), then the weight-streaming path on the same scratch
    (Workload("na_tiled", 600, 256, 384, 4, 2, 6, 16),
     Workload("na_tiled_small", 40, 256, 384, 4, 2, 6, 16)),
])
def test_noalloc_equals_forward_twice(big, small):
    for w in (big, small):
        _say(f"noalloc {w.name} T={w.T}")
        inp, y_ref, y_na = _pair(w, 11)
        assert torch.equal(y_na, y_ref), f"{w.name}: differs from moe_lora_forward"
        check_close(y_na, oracle_rows(inp, w.topk), what=f"noalloc {w.name}")


def test_noalloc_full_size_decode_then_tiny():
    """The decode batch (27 MiB of workspace) and then the tiny one, on the same scratch."""
    w = configs.WORKLOADS["decode"]
    _say("noalloc decode")
    inp = configs.make_inputs(w, 2, device=DEV)
    keys = ("x", "logits", "W1", "W2", "A1", "B1", "A2", "B2", "adapter_ids")
    y_ref = ml.forward(*[inp[k] for k in keys], w.topk)
    y_na = ml.forward_noalloc(*[inp[k] for k in keys], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ref)
    del inp
    torch.cuda.empty_cache()
    t = configs.WORKLOADS["tiny"]
    _say("noalloc tiny")
    inp, y_ref, y_na = _pair(t, 3)
    assert torch.equal(y_na, y_ref)
    check_close(y_na, oracle_rows(inp, t.topk), what="noalloc tiny")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    w = configs.WORKLOADS["prefill"]
    d = ml.Dims(w.T, w.hidden, w.inter, w.n_experts, w.n_adapters, w.rank)
    assert ml.workspace_size(d, w.topk) > 128 << 20
    x = torch.zeros(1, dtype=torch.bfloat16, device=DEV)  # never read: the size check comes first
    args = [x.data_ptr()] * 9
    rc = ml.lib().moe_lora_forward_noalloc(*args, w.topk, ml.ctypes.byref(d), x.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == ml.ESCRATCH

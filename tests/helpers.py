"""Shared test helpers: sampled-token oracle evaluation for inputs that live on the GPU, and
the tolerance checks. Expected values always come from oracle/ on host copies of the inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = 2e-2  # max |y - y_ref| <= TOL * max |y_ref|, globally and per token


def sample_tokens(T: int, n: int = 12, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(np.arange(1, T - 1), n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(picks), dtype=np.int32)


def oracle_rows(inp: dict, topk: int, tokens=None) -> np.ndarray:
    """Oracle y (float64) for `tokens` (all when None). Inputs may be on the GPU: only the
    tokens' rows and the adapters they use are copied to the host (adapter ids remapped)."""
    x = inp["x"]
    T = x.shape[0]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tok_t = torch.as_tensor(np.asarray(tokens, dtype=np.int64), device=x.device)
    ad = inp["adapter_ids"].index_select(0, tok_t).cpu().numpy().astype(np.int32)
    nA = inp["A1"].shape[0]
    used = sorted({int(a) for a in ad if 0 <= a < nA}) or [0]
    remap = {a: i for i, a in enumerate(used)}
    ad_new = np.array([remap.get(int(a), -1) for a in ad], dtype=np.int32)
    used_t = torch.as_tensor(used, dtype=torch.int64, device=x.device)
    host = {
        "x": x.index_select(0, tok_t).cpu(),
        "logits": inp["logits"].index_select(0, tok_t).cpu(),
        "adapter_ids": ad_new,
        "W1": inp["W1"].cpu(),
        "W2": inp["W2"].cpu(),
    }
    for name in ("W1_scale", "W2_scale"):  # E4M3 weights: per-row scales
        if name in inp:
            host[name] = inp[name].cpu()
    for name in ("A1", "B1", "A2", "B2"):
        host[name] = inp[name].index_select(0, used_t).cpu()
    return oracle.forward(host, topk)


def expected_layout(logits, adapter_ids, topk: int, n_experts: int, n_adapters: int, block_m: int) -> dict:
    """The routing and sorted-layout tables a layer call must produce at row blocks of block_m
    (seg_pad 1), from the oracle's route and align; the per-block and per-row tables follow from
    those by their definitions (expert of the padded region holding the block's first row,
    segment holding it or -1 for padding, inverse of the sorted order, adapter of the row's
    token or -1)."""
    L = logits.cpu() if isinstance(logits, torch.Tensor) else torch.from_numpy(np.asarray(logits))
    ad = (adapter_ids.cpu().numpy() if isinstance(adapter_ids, torch.Tensor)
          else np.asarray(adapter_ids)).astype(np.int32)
    ids, w = oracle.route(L, topk)
    al = oracle.align(ids, ad, n_experts, n_adapters, 1, block_m)
    sp, off, seg = al["sorted_pairs"], al["expert_offsets"], al["seg_table"]
    total = len(sp)
    assert total % block_m == 0
    n_blocks = total // block_m
    rows0 = np.arange(n_blocks, dtype=np.int64) * block_m
    block_expert = (np.searchsorted(off, rows0, side="right") - 1).astype(np.int32)
    block_seg = np.full(n_blocks, -1, np.int32)
    for s, (_, _, st, cnt) in enumerate(seg):
        b_lo = -(-int(st) // block_m)
        for b in range(b_lo, n_blocks):
            if b * block_m >= st + cnt:
                break
            block_seg[b] = s
    real = sp >= 0
    pair_row = np.full(ids.size, -1, np.int32)
    pair_row[sp[real]] = np.nonzero(real)[0].astype(np.int32)
    sorted_ad = np.full(total, -1, np.int32)
    sorted_ad[real] = ad[sp[real] // topk]
    return {"topk_ids": ids, "topk_w": w.astype(np.float32), "sorted_pairs": sp,
            "expert_offsets": off, "seg_table": seg, "n_blocks": n_blocks,
            "block_expert": block_expert, "block_seg": block_seg, "pair_row": pair_row,
            "sorted_ad": sorted_ad}


def check_close(y_gpu: torch.Tensor, y_ref: np.ndarray, tol: float = TOL, what: str = ""):
    y = y_gpu.double().cpu().numpy()
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    gmax = np.abs(y_ref).max()
    assert err.max() <= tol * gmax, f"{what}: max err {err.max():.3e} > {tol} * {gmax:.3e}"
    per_tok = err.max(axis=1)
    bound = tol * np.abs(y_ref).max(axis=1)
    bad = np.nonzero(per_tok > bound)[0]
    assert bad.size == 0, f"{what}: tokens {bad[:8].tolist()} exceed the per-token bound"
    return float(err.max() / gmax) if gmax > 0 else 0.0

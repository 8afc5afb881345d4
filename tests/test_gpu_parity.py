"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Routing ids, slot order, sorted pairs, expert offsets and the segment table must match
bit for bit; y must satisfy max|y - y_ref| <= 2e-2 * max|y_ref| globally and per token."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import lora_mixture_experts_amd as ml
import oracle
from synth import configs
from synth.configs import Workload
from tests.helpers import check_close, expected_layout, oracle_rows, sample_tokens

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _dims(w: Workload) -> ml.Dims:
    return ml.Dims(w.T, w.hidden, w.inter, w.n_experts, w.n_adapters, w.rank)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------- route + align

# (seg_pad, block_m) settings: every one the forward uses (seg_pad 1 with 16-, 32-, 64-, 128-, 192-
# and 256-row blocks) and a few with padded segments
ROUTE_CASES = [
    ("tiny", 1, 1), ("tiny", 4, 16), ("decode", 1, 16), ("decode", 16, 16), ("prefill", 1, 64),
    ("prefill", 16, 128), ("fg", 1, 32), ("fg", 8, 32), ("stress_distinct", 1, 64),
    ("stress_same", 1, 64), ("stress_distinct", 16, 256), ("prefill", 1, 256), ("prefill", 1, 128),
    ("stress_distinct", 1, 128), ("stress_same", 1, 256), ("fg", 1, 16), ("tiny", 1, 128),
    ("stress_distinct", 1, 192), ("stress_same", 1, 192), ("tiny", 3, 192),
]


def _route_align_case(w: Workload, L: torch.Tensor, ad: torch.Tensor, seg_pad: int, block_m: int):
    _say(f"route_align {w.name} T={w.T} E={w.n_experts} k={w.topk} nA={w.n_adapters} "
         f"seg_pad={seg_pad} block_m={block_m}")
    d = _dims(w)
    out = ml.route_align(L.to(DEV), ad.to(DEV), w.topk, d, seg_pad, block_m)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route(L, w.topk)
    al = oracle.align(ids_ref, ad.numpy(), w.n_experts, w.n_adapters, seg_pad, block_m)
    np.testing.assert_array_equal(out["topk_ids"].cpu().numpy(), ids_ref)
    np.testing.assert_allclose(out["topk_w"].cpu().numpy(), w_ref, rtol=0, atol=2e-6)
    total = int(al["expert_offsets"][-1])
    np.testing.assert_array_equal(out["expert_offsets"].cpu().numpy(), al["expert_offsets"])
    sp = out["sorted_pairs"].cpu().numpy()
    np.testing.assert_array_equal(sp[:total], al["sorted_pairs"])
    assert np.all(sp[total:] == -7), "wrote past the padded total"
    assert int(out["n_seg"].item()) == al["n_seg"]
    np.testing.assert_array_equal(out["seg_table"].cpu().numpy()[: al["n_seg"]], al["seg_table"])
    assert ml.debug_status(out["workspace"]) == 0


@pytest.mark.parametrize("name,seg_pad,block_m", ROUTE_CASES)
def test_route_align_bit_exact(name, seg_pad, block_m):
    w = configs.WORKLOADS[name]
    _route_align_case(w, configs.make_logits(w, 0), configs.make_adapter_ids(w, 0), seg_pad, block_m)


# E up to 256 takes the rank-count routing kernel, larger E the arg-max rounds
@pytest.mark.parametrize("E,k,levels", [(8, 2, 2), (128, 8, 3), (16, 16, 1), (1, 1, 1), (200, 5, 2),
                                        (256, 16, 3), (300, 6, 2), (1000, 3, 4)])
def test_route_align_ties_and_no_adapter(E, k, levels):
    w = Workload("ties", 300, 128, 128, E, k, 7, 8)
    rng = np.random.default_rng(E + k)
    L = np.round(rng.standard_normal((w.T, E)) * levels / 2) / levels
    L = L.astype(np.float32)
    L[L == 0] = np.where(rng.random(int((L == 0).sum())) < 0.5, -0.0, 0.0)
    ad = rng.integers(-1, 7, w.T).astype(np.int32)
    _route_align_case(w, torch.from_numpy(L), torch.from_numpy(ad), 4, 32)


@pytest.mark.parametrize("T,E,k,nA", [(512, 64, 4, 1000), (20000, 16, 2, 4), (3000, 200, 6, 300)])
def test_route_align_large_tables(T, E, k, nA):
    """Bucket tables or staged inputs too large for LDS take the workspace path."""
    w = Workload("big", T, 128, 128, E, k, nA, 8)
    L = configs.make_logits(w, 3)
    ad = torch.from_numpy(np.random.default_rng(T).integers(-1, nA, T).astype(np.int32))
    _route_align_case(w, L, ad, 1, 64)


def test_route_align_empty():
    w = Workload("empty", 0, 128, 128, 8, 2, 3, 8)
    out = ml.route_align(torch.zeros((0, 8), device=DEV), torch.zeros(0, dtype=torch.int32, device=DEV),
                         2, _dims(w), 1, 16)
    torch.cuda.synchronize()
    assert out["expert_offsets"].cpu().tolist() == [0] * 9
    assert int(out["n_seg"].item()) == 0


# ----------------------------------------------------------------------------- forward, small shapes

SMALL = {
    "tiny": configs.WORKLOADS["tiny"],
    "ragged": Workload("ragged", 37, 384, 640, 6, 2, 5, 16),
    "r8_k1": Workload("r8_k1", 23, 256, 256, 4, 1, 3, 8),
    "r32_k4": Workload("r32_k4", 50, 512, 384, 16, 4, 7, 32),
    "r64_E1": Workload("r64_E1", 19, 256, 512, 1, 1, 3, 64),
    "mid": Workload("mid", 200, 256, 384, 8, 2, 6, 16),
    "fg_small": Workload("fg_small", 64, 256, 256, 32, 8, 16, 32, hot_experts=4, hot_bias=2.0),
    "one_token": Workload("one_token", 1, 256, 384, 8, 2, 4, 16),
    # mean rows per expert above 24 selects the LDS-tiled MFMA path: 64-row blocks below 192
    # rows per expert, 128-row blocks below 768
    "tiled64": Workload("tiled64", 256, 384, 640, 4, 2, 5, 16),
    "tiled64_r8": Workload("tiled64_r8", 300, 256, 256, 4, 1, 3, 8),
    "tiled128_r64": Workload("tiled128_r64", 900, 256, 384, 3, 2, 6, 64),
    "tiled128_runs": Workload("tiled128_runs", 1024, 256, 256, 4, 2, 9, 32, adapters="zipf_runs", run=40),
    "tiled128_h384": Workload("tiled128_h384", 1600, 384, 640, 2, 1, 4, 16),  # 256 tiles do not divide h
    # 768 rows per expert and more, with 2I and h multiples of 256, selects 256x256 tiles
    "tiled256_r64": Workload("tiled256_r64", 2048, 256, 384, 4, 2, 6, 64, adapters="zipf_runs", run=100),
    "tiled256_k1": Workload("tiled256_k1", 1600, 512, 640, 2, 1, 4, 16),
    "tiled256_shortk": Workload("tiled256_shortk", 1700, 256, 128, 3, 2, 4, 16),  # down: 2 K steps
    # about 100 to 160 rows per expert: 192-row layout blocks, gate_up in 64-row sub-tiles (tiles
    # of padding only skipped), down in 192-row tiles
    "tiled192": Workload("tiled192", 512, 256, 384, 8, 2, 6, 16),
    "tiled192_distinct": Workload("tiled192_distinct", 600, 256, 256, 8, 2, 600, 16, adapters="distinct"),
}


def _small_inputs(w: Workload, seed: int, b_scale=1.0, no_adapter_every=5):
    inp = configs.make_inputs(w, seed, b_scale=b_scale)
    if no_adapter_every:
        inp["adapter_ids"][::no_adapter_every] = -1
    return inp


def _run(inp: dict, topk: int, workspace=None):
    g = {k: v.to(DEV) for k, v in inp.items()}
    y = ml.forward(g["x"], g["logits"], g["W1"], g["W2"], g["A1"], g["B1"], g["A2"], g["B2"],
                   g["adapter_ids"], topk, workspace=workspace)
    torch.cuda.synchronize()
    return y


def check_forward_tables(ws: torch.Tensor, w: Workload, logits, adapter_ids):
    """The forward's own routing and sorted-layout tables in its workspace, bit for bit against
    the oracle's routing and align at the row-block size the call used (seg_pad 1), and the
    derived tables (row block -> expert and first segment, pair -> row, row -> adapter)."""
    d = _dims(w)
    got = ml.read_layout_tables(ws, d, w.topk)
    bm = got["info"]["block_m"]
    ref = expected_layout(logits, adapter_ids, w.topk, w.n_experts, w.n_adapters, bm)
    np.testing.assert_array_equal(got["topk_ids"], ref["topk_ids"])
    np.testing.assert_allclose(got["topk_w"], ref["topk_w"], rtol=0, atol=2e-6)
    assert got["n_blocks"] == ref["n_blocks"], (got["n_blocks"], ref["n_blocks"])
    for key in ("sorted_pairs", "expert_offsets", "seg_table", "block_expert", "block_seg", "pair_row",
                "sorted_ad"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{w.name}: {key} (block_m {bm})")
    return got


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_layout_tables_bit_exact(name):
    w = SMALL[name]
    _say(f"forward tables {name}")
    inp = _small_inputs(w, 1)
    ws = ml.new_workspace(_dims(w), w.topk, DEV)
    _run(inp, w.topk, workspace=ws)
    check_forward_tables(ws, w, inp["logits"], inp["adapter_ids"])


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("b_scale", [1.0, 10.0])
def test_forward_small_vs_oracle(name, b_scale):
    w = SMALL[name]
    _say(f"forward {name} b_scale={b_scale}")
    inp = _small_inputs(w, 1, b_scale)
    y = _run(inp, w.topk)
    y_ref = oracle_rows(inp, w.topk)
    check_close(y, y_ref, what=f"{name} b_scale={b_scale}")


def test_forward_all_adapters_off_and_on():
    w = SMALL["ragged"]
    inp = _small_inputs(w, 2, 10.0, no_adapter_every=0)
    off = dict(inp)
    off["adapter_ids"] = torch.full_like(inp["adapter_ids"], -1)
    y_off = _run(off, w.topk)
    check_close(y_off, oracle_rows(off, w.topk), what="adapters off")
    y_on = _run(inp, w.topk)
    ref_on = oracle_rows(inp, w.topk)
    check_close(y_on, ref_on, what="adapters on")
    # the LoRA terms are visible at this scale: the adapter-free output must not pass as it
    assert np.abs(y_off.double().cpu().numpy() - ref_on).max() > 0.1 * np.abs(ref_on).max()


def test_forward_tiled_mixed_run_lengths():
    """Long adapter runs (64-row shrink) next to one adapter per token (segment shrink) in the
    same batch, on 256-row tiles: every 64-row sub-block is taken by exactly one of the two
    shrinks, and a segment that crosses into a sub-block of long runs leaves its rows there."""
    w = Workload("tiled256_mixed", 2048, 256, 384, 4, 2, 40, 32, adapters="zipf_runs", run=128)
    _say("forward tiled256_mixed")
    inp = _small_inputs(w, 3, 10.0, no_adapter_every=0)
    g = torch.Generator().manual_seed(3)
    inp["adapter_ids"][w.T // 2:] = torch.randint(-1, w.n_adapters, (w.T - w.T // 2,), generator=g,
                                                  dtype=torch.int32)
    y = _run(inp, w.topk)
    check_close(y, oracle_rows(inp, w.topk), what="tiled256_mixed")


def test_forward_empty_batch():
    w = SMALL["tiny"].with_(T=0)
    inp = configs.make_inputs(w, 0)
    y = _run(inp, w.topk)
    assert y.shape == (0, w.hidden)


def test_forward_flags_bad_adapter_and_nonfinite_logit():
    w = SMALL["ragged"]
    inp = _small_inputs(w, 3, 10.0)
    bad = dict(inp)
    bad["adapter_ids"] = inp["adapter_ids"].clone()
    bad["adapter_ids"][4] = w.n_adapters + 3
    g = {k: v.to(DEV) for k, v in bad.items()}
    ws = ml.new_workspace(_dims(w), w.topk, DEV)
    y = ml.forward(g["x"], g["logits"], g["W1"], g["W2"], g["A1"], g["B1"], g["A2"], g["B2"],
                   g["adapter_ids"], w.topk, workspace=ws)
    assert ml.debug_status(ws) == ml.FLAG_ADAPTER_RANGE
    as_none = dict(inp)
    as_none["adapter_ids"] = bad["adapter_ids"].clone()
    as_none["adapter_ids"][4] = -1
    check_close(y, oracle_rows(as_none, w.topk), what="out-of-range adapter acts as none")

    nf = dict(inp)
    nf["logits"] = inp["logits"].clone()
    nf["logits"][6, 1] = float("nan")
    g = {k: v.to(DEV) for k, v in nf.items()}
    y = ml.forward(g["x"], g["logits"], g["W1"], g["W2"], g["A1"], g["B1"], g["A2"], g["B2"],
                   g["adapter_ids"], w.topk, workspace=ws)
    assert ml.debug_status(ws) == ml.FLAG_NONFINITE_LOGIT
    keep = np.array([t for t in range(w.T) if t != 6], np.int32)
    check_close(y[torch.from_numpy(keep).long().to(DEV)], oracle_rows(inp, w.topk, keep), what="finite tokens")


@pytest.mark.parametrize("name", ["fg_small", "tiled64", "tiled256_r64", "tiled128_runs", "tiled192"])
def test_forward_poisoned_workspace_and_determinism(name):
    """Whatever the workspace held before (all-ones bytes, 0x7F bytes, a fresh allocation), the
    call gives the same bytes, within the bound of the oracle: no stage reads a region it did not
    write first (z planes, act, the down split parts, align tables)."""
    w = SMALL[name]
    _say(f"poisoned workspace {name}")
    inp = _small_inputs(w, 4)
    ws = ml.new_workspace(_dims(w), w.topk, DEV)
    ws.fill_(0xFF)
    y1 = _run(inp, w.topk, workspace=ws).clone()
    ws.fill_(0x7F)
    y2 = _run(inp, w.topk, workspace=ws).clone()
    y3 = _run(inp, w.topk)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    check_close(y1, oracle_rows(inp, w.topk), what="poisoned workspace")


# ----------------------------------------------------------------------------- full-size configs

def _all_tokens_chunked(inp, w, y, what, chunk=256):
    """y against the oracle on every token, a chunk of tokens at a time (only the adapters a
    chunk uses are copied to the host)."""
    worst = 0.0
    for t0 in range(0, w.T, chunk):
        toks = np.arange(t0, min(w.T, t0 + chunk), dtype=np.int32)
        y_ref = oracle_rows(inp, w.topk, toks)
        worst = max(worst, check_close(y[torch.from_numpy(toks).long().to(DEV)], y_ref,
                                       what=f"{what} tokens {t0}..{toks[-1]}"))
    return worst


def _block_tokens(tables, topk: int, sub: int = 64) -> np.ndarray:
    """Tokens of the first and last real row of every `sub`-row sub-block of the sorted layout
    (so every row block of every expert, every 64-row shrink sub-block and every column tile of
    those rows is compared), plus the batch's first and last token."""
    sp = tables["sorted_pairs"]
    toks = set()
    for b0 in range(0, len(sp), sub):
        real = sp[b0:b0 + sub]
        real = real[real >= 0]
        if real.size:
            toks.add(int(real[0]) // topk)
            toks.add(int(real[-1]) // topk)
    return np.array(sorted(toks), dtype=np.int32)


def _full_case(name: str, seed: int = 0, b_scale: float = 1.0, adapters=None):
    """Full-size layer call: its routing tables bit for bit, then y against the oracle on every
    token (prefill: two tokens per 64-row sub-block of the sorted layout)."""
    w = configs.WORKLOADS[name]
    _say(f"full-size {name}: generating inputs on the GPU")
    inp = configs.make_inputs(w, seed, device=DEV, b_scale=b_scale)
    if adapters is not None:
        inp["adapter_ids"] = adapters
    ws = ml.new_workspace(_dims(w), w.topk, DEV)
    _say(f"full-size {name}: forward")
    y = ml.forward(inp["x"], inp["logits"], inp["W1"], inp["W2"], inp["A1"], inp["B1"], inp["A2"],
                   inp["B2"], inp["adapter_ids"], w.topk, workspace=ws)
    torch.cuda.synchronize()
    tables = check_forward_tables(ws, w, inp["logits"].cpu(), inp["adapter_ids"].cpu())
    if w.T <= 1024:
        _say(f"full-size {name}: oracle on all {w.T} tokens")
        rel = _all_tokens_chunked(inp, w, y, name)
    else:
        toks = _block_tokens(tables, w.topk)
        _say(f"full-size {name}: oracle on {len(toks)} tokens covering every 64-row sub-block")
        rel = check_close(y[torch.from_numpy(toks).long().to(DEV)], oracle_rows(inp, w.topk, toks),
                          what=name)
    _say(f"full-size {name}: max rel err {rel:.2e}")
    return inp, y, ws


@pytest.mark.parametrize("name", ["decode", "prefill", "fg"])
def test_forward_full_size(name):
    inp, y, ws = _full_case(name)
    # the same call again, on the same workspace, gives the same bytes
    w = configs.WORKLOADS[name]
    y2 = ml.forward(inp["x"], inp["logits"], inp["W1"], inp["W2"], inp["A1"], inp["B1"], inp["A2"],
                    inp["B2"], inp["adapter_ids"], w.topk, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    del inp, ws
    torch.cuda.empty_cache()


def test_forward_full_size_decode_amplified_b():
    _full_case("decode", seed=1, b_scale=10.0)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["stress_distinct", "stress_same"])
def test_forward_full_size_stress(name):
    """The adapter-diversity batch with every token on its own adapter, and the same batch with
    every token on adapter 0: every token of both against the oracle."""
    _full_case(name)
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- FP8 expert weights

# every small shape: the weight-streaming ones (at most 24 token-expert pairs per expert) and the
# LDS-tiled ones (64-, 128- and 256-row blocks)
FP8_SMALL = list(SMALL)


def _run_fp8(inp: dict, topk: int, workspace=None):
    g = {k: v.to(DEV) for k, v in inp.items()}
    y = ml.forward_fp8(g["x"], g["logits"], g["W1"], g["W1_scale"], g["W2"], g["W2_scale"],
                       g["A1"], g["B1"], g["A2"], g["B2"], g["adapter_ids"], topk,
                       workspace=workspace)
    torch.cuda.synchronize()
    return y


def test_fp8_small_cases_cover_both_paths():
    tiled = {n for n in FP8_SMALL if SMALL[n].T * SMALL[n].topk > 24 * SMALL[n].n_experts}
    assert {"tiny", "ragged", "r8_k1", "r32_k4", "r64_E1", "fg_small", "one_token"} <= set(FP8_SMALL)
    assert {"tiled64", "tiled128_r64", "tiled256_r64", "tiled256_shortk"} <= tiled


@pytest.mark.parametrize("name", FP8_SMALL)
@pytest.mark.parametrize("b_scale", [1.0, 10.0])
def test_forward_fp8_small_vs_oracle(name, b_scale):
    w = SMALL[name]
    _say(f"forward fp8 {name} b_scale={b_scale}")
    inp = configs.make_inputs_fp8(w, 3, b_scale=b_scale)
    inp["adapter_ids"][::5] = -1
    y = _run_fp8(inp, w.topk)
    check_close(y, oracle_rows(inp, w.topk), what=f"fp8 {name} b_scale={b_scale}")


@pytest.mark.parametrize("name", ["ragged", "tiled64", "tiled256_r64"])
def test_forward_fp8_scales_matter(name):
    """Doubling one expert's scales doubles its base term: the output changes where the oracle
    says it does (a kernel that ignored the scales, or applied them to the wrong rows, fails)."""
    w = SMALL[name]
    inp = configs.make_inputs_fp8(w, 4)
    inp["W1_scale"][1] *= 2.0
    inp["W2_scale"][0, : w.hidden // 2] *= 0.5
    y = _run_fp8(inp, w.topk)
    check_close(y, oracle_rows(inp, w.topk), what=f"fp8 rescaled experts {name}")


@pytest.mark.parametrize("name", ["decode", "fg", "stress_same", "prefill"])
def test_forward_fp8_full_size(name):
    w = configs.WORKLOADS[name]
    _say(f"full-size fp8 {name}: generating inputs on the GPU")
    inp = configs.make_inputs_fp8(w, 0, device=DEV)
    _say(f"full-size fp8 {name}: forward")
    args = (inp["x"], inp["logits"], inp["W1"], inp["W1_scale"], inp["W2"], inp["W2_scale"],
            inp["A1"], inp["B1"], inp["A2"], inp["B2"], inp["adapter_ids"], w.topk)
    y = ml.forward_fp8(*args)
    torch.cuda.synchronize()
    if w.T <= 1024:
        _say(f"full-size fp8 {name}: oracle on all {w.T} tokens")
        rel = _all_tokens_chunked(inp, w, y, f"fp8 {name}")
    else:
        ws = ml.new_workspace(_dims(w), w.topk, DEV)
        ml.forward_fp8(*args, workspace=ws)
        torch.cuda.synchronize()
        toks = _block_tokens(ml.read_layout_tables(ws, _dims(w), w.topk), w.topk)
        del ws
        _say(f"full-size fp8 {name}: oracle on {len(toks)} tokens covering every 64-row sub-block")
        rel = check_close(y[torch.from_numpy(toks).long().to(DEV)], oracle_rows(inp, w.topk, toks),
                          what=f"fp8 {name}")
    _say(f"full-size fp8 {name}: max rel err {rel:.2e}")
    y2 = ml.forward_fp8(*args)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    del inp
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- HIP graph capture

@pytest.mark.parametrize("name", ["ragged", "tiled64", "fg_small"])
def test_forward_graph_capture_replays(name):
    """One layer call captured in a HIP graph (the library enqueues kernels only: no memset,
    no host synchronisation) and replayed several times, with other eager calls on the same
    workspace in between: every replay equals the eager result."""
    w = SMALL[name]
    inp = {k: v.to(DEV) for k, v in _small_inputs(w, 6).items()}
    other = {k: v.to(DEV) for k, v in _small_inputs(w, 7).items()}
    d = ml.Dims(w.T, w.hidden, w.inter, w.n_experts, w.n_adapters, w.rank)
    ws = ml.new_workspace(d, w.topk, DEV)
    y = torch.empty((w.T, w.hidden), dtype=torch.bfloat16, device=DEV)
    y_other = torch.empty_like(y)
    keys = ("x", "logits", "W1", "W2", "A1", "B1", "A2", "B2", "adapter_ids")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ml.forward(*[inp[k] for k in keys], w.topk, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    y_eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ml.forward(*[inp[k] for k in keys], w.topk, y=y, workspace=ws)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(0)
        ml.forward(*[other[k] for k in keys], w.topk, y=y_other, workspace=ws)  # eager, same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
    check_close(y, oracle_rows(inp, w.topk), what=f"graph replay {name}")


# ----------------------------------------------------------------------------- dense multi-LoRA

SGMV_CASES = [
    # T, K, N, nA, r, adapters
    (37, 256, 192, 5, 16, "uniform"),
    (1, 128, 64, 3, 8, "uniform"),
    (200, 512, 320, 64, 32, "uniform"),
    (300, 384, 256, 4, 64, "runs"),
    (64, 256, 128, 1, 16, "same"),
    (700, 256, 256, 700, 16, "distinct"),
    (2000, 128, 64, 8, 8, "runs"),
    # the one-workgroup adapter sort's limits (1024 tokens, 1024 adapters) and just past them
    (1024, 256, 128, 1024, 8, "distinct"),
    (1025, 128, 64, 5, 16, "uniform"),
    (1000, 128, 64, 1100, 8, "uniform"),
]


def _sgmv_case(T, K, N, nA, r, adapters, seed):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(T, K, generator=g) * 0.5).to(torch.bfloat16)
    A = (torch.randn(nA, r, K, generator=g) * 0.05).to(torch.bfloat16)
    B = (torch.randn(nA, N, r, generator=g) * 0.05).to(torch.bfloat16)
    if adapters == "uniform":
        ad = torch.randint(-1, nA, (T,), generator=g, dtype=torch.int32)
    elif adapters == "runs":
        ad = (torch.arange(T, dtype=torch.int32) // 41) % nA
        ad[::7] = -1
    elif adapters == "same":
        ad = torch.zeros(T, dtype=torch.int32)
    else:
        ad = torch.randperm(nA, generator=g)[:T].to(torch.int32)
    return x, A, B, ad


@pytest.mark.parametrize("T,K,N,nA,r,adapters", SGMV_CASES)
def test_sgmv_vs_oracle(T, K, N, nA, r, adapters):
    _say(f"sgmv T={T} K={K} N={N} nA={nA} r={r} {adapters}")
    x, A, B, ad = _sgmv_case(T, K, N, nA, r, adapters, T + nA)
    # onto y = 0: the LoRA term alone, against the oracle's; untouched tokens stay exactly 0
    y = torch.zeros(T, N, dtype=torch.bfloat16, device=DEV)
    ml.sgmv(x.to(DEV), A.to(DEV), B.to(DEV), ad.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.sgmv(x, A, B, torch.zeros(T, N, dtype=torch.bfloat16), ad)
    check_close(y, ref, what="sgmv term")
    none = (ad < 0).numpy()
    assert np.all(y.float().cpu().numpy()[none] == 0)
    # onto a given y: within one bf16 rounding of the sum, tokens without adapter bit-exact
    y0 = torch.randn(T, N, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    y = y0.to(DEV)
    ml.sgmv(x.to(DEV), A.to(DEV), B.to(DEV), ad.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.sgmv(x, A, B, y0, ad)
    got = y.double().cpu().numpy()
    term = np.abs(ref - y0.double().numpy()).max()
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-2 * term)
    assert torch.equal(y.cpu()[torch.from_numpy(none)], y0[torch.from_numpy(none)])


def test_sgmv_empty_and_bad_adapters():
    x, A, B, ad = _sgmv_case(50, 128, 64, 3, 8, "uniform", 9)
    ad[::4] = 17  # out of range: no adapter, flag set
    d = ml.SgmvDims(50, 128, 64, 3, 8)
    ws = torch.empty(int(ml.lib().moe_lora_sgmv_workspace_size(ctypes.byref(d))), dtype=torch.uint8,
                     device=DEV)
    y = torch.zeros(50, 64, dtype=torch.bfloat16, device=DEV)
    ml.sgmv(x.to(DEV), A.to(DEV), B.to(DEV), ad.to(DEV), y, workspace=ws)
    torch.cuda.synchronize()
    ad_ref = torch.where(ad >= 3, torch.full_like(ad, -1), ad)
    check_close(y, oracle.sgmv(x, A, B, torch.zeros(50, 64, dtype=torch.bfloat16), ad_ref),
                what="sgmv bad adapters")
    assert ml.debug_status(ws) == ml.FLAG_ADAPTER_RANGE
    e = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    ml.sgmv(x[:0].to(DEV), A.to(DEV), B.to(DEV), ad[:0].to(DEV), e)


# ----------------------------------------------------------------------------- router GEMM

@pytest.mark.parametrize("T,h,E", [(37, 256, 8), (64, 4096, 16), (256, 2048, 128), (1, 128, 1),
                                   (300, 384, 200), (4096, 4096, 8), (16, 8192, 32), (5, 640, 3)])
def test_router_logits_vs_oracle(T, h, E):
    """fp32 logits within a rounding bound of the float64 dot products: 3e-5 of the sum of the
    products' magnitudes (a dropped or wrong K chunk moves a logit by far more)."""
    g = torch.Generator().manual_seed(T + E)
    x = torch.randn(T, h, generator=g).to(torch.bfloat16)
    W = (torch.randn(E, h, generator=g) * 0.02).to(torch.bfloat16)
    got = ml.router_logits(x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.router_logits(x, W)
    bound = 3e-5 * (np.abs(x.double().numpy()) @ np.abs(W.double().numpy()).T) + 1e-30
    err = np.abs(got.cpu().double().numpy() - ref)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("name", ["ragged", "fg_small", "tiled64"])
def test_forward_routed_equals_forward_on_its_logits(name):
    """The layer from router weights equals the layer on the router kernel's logits, bit for
    bit, and routing on those fp32 logits matches the oracle's selection on the same values."""
    w = SMALL[name]
    inp = {k: v.to(DEV) for k, v in _small_inputs(w, 8).items()}
    Wr = (torch.randn(w.n_experts, w.hidden, generator=torch.Generator().manual_seed(5)) * 0.5).to(
        torch.bfloat16).to(DEV)
    keys = ("W1", "W2", "A1", "B1", "A2", "B2", "adapter_ids")
    y_r = ml.forward_routed(inp["x"], Wr, *[inp[k] for k in keys], w.topk)
    logits = ml.router_logits(inp["x"], Wr)
    y_f = ml.forward(inp["x"], logits, *[inp[k] for k in keys], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(y_r, y_f)
    ra = ml.route_align(logits, inp["adapter_ids"], w.topk, _dims(w), 1, 1)
    torch.cuda.synchronize()
    ids_ref, _ = oracle.route(logits.cpu(), w.topk)
    np.testing.assert_array_equal(ra["topk_ids"].cpu().numpy(), ids_ref)
    host = {k: v.cpu() for k, v in inp.items()}
    host["logits"] = logits.cpu()
    check_close(y_r, oracle_rows(host, w.topk), what=f"routed {name}")

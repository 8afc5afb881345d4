"""Pins of the float64 CPU oracle against facts that do not come from the oracle itself:
hand-worked fixtures, Python's own sort, scipy's softmax, numpy matmul, and exact
identities of the method (merged weights, B = 0, per-token evaluation, permutations,
linearity). CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from synth import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64_inputs(w, seed, b_scale=1.0):
    d = configs.make_inputs(w, seed, dtype=torch.float64, b_scale=b_scale)
    return {k: (v.numpy() if hasattr(v, "numpy") else v) for k, v in d.items()}


TINY = configs.WORKLOADS["tiny"]


def _ffn_numpy(x, W1, W2, A1, B1, A2, B2, a):
    """Dense SwiGLU FFN with LoRA for rows x, computed with numpy matmul."""
    I = W1.shape[0] // 2
    g = x @ W1.T
    if a >= 0:
        g = g + (x @ A1.T) @ B1.T
    act = g[:, :I] / (1.0 + np.exp(-g[:, :I])) * g[:, I:]
    d = act @ W2.T
    if a >= 0:
        d = d + (act @ A2.T) @ B2.T
    return d


# ----------------------------------------------------------------------------- route

def test_route_golden_ties():
    g = json.load(open(os.path.join(GOLDEN, "route_ties.json")))
    L = np.array([g["logits"]], np.float32)
    ids, w = oracle.route(L, g["k"])
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], g["w"], rtol=0, atol=g["tol"])


@pytest.mark.parametrize("E,k,levels", [(8, 2, None), (8, 2, 3), (16, 2, None), (128, 8, None),
                                        (128, 8, 5), (5, 5, 2), (1, 1, None)])
def test_route_vs_python_sort(E, k, levels):
    rng = np.random.default_rng(E * 100 + k)
    T = 64
    L = rng.standard_normal((T, E)).astype(np.float32)
    if levels:  # force many exact ties, including signed zeros
        L = (np.round(L * levels / 3) / levels).astype(np.float32)
        L[L == 0] = np.where(rng.random((L == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    ids, w = oracle.route(L, k)
    for t in range(T):
        expect = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k]
        assert ids[t].tolist() == expect
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


@pytest.mark.parametrize("name", ["decode", "prefill", "fg", "stress_distinct"])
def test_route_full_size_vs_python_sort(name):
    w = configs.WORKLOADS[name]
    L = configs.make_logits(w, 0).numpy()
    ids, _ = oracle.route(L, w.topk)
    order = np.lexsort((np.broadcast_to(np.arange(w.n_experts), L.shape), -L.astype(np.float64)), axis=1)
    np.testing.assert_array_equal(ids, order[:, : w.topk])


def test_route_k1_and_kE_weights():
    rng = np.random.default_rng(7)
    L = rng.standard_normal((32, 6)).astype(np.float32)
    _, w1 = oracle.route(L, 1)
    assert np.all(w1 == 1.0)
    ids, wE = oracle.route(L, 6)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(wE, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13, atol=0)


def test_route_rejects_nonfinite():
    L = np.zeros((2, 4), np.float32)
    L[1, 2] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.route(L, 2)


# ----------------------------------------------------------------------------- align

def _check_align(ids, ad, E, nA, seg_pad, block_m):
    T, k = ids.shape
    out = oracle.align(ids, ad, E, nA, seg_pad, block_m)
    sp, off, seg = out["sorted_pairs"], out["expert_offsets"], out["seg_table"]
    real = sp[sp >= 0]
    # every pair exactly once
    assert sorted(real.tolist()) == list(range(T * k))
    # order equals Python's sort on the key (e, a, t)
    keys = [(int(ids.reshape(-1)[p]), int(ad[p // k]), p // k) for p in range(T * k)]
    expect = sorted(range(T * k), key=lambda p: keys[p])
    assert real.tolist() == expect
    # expert blocks: offsets, alignment, per-expert counts
    cnt_e = np.bincount(ids.reshape(-1), minlength=E)
    assert off[0] == 0
    for e in range(E):
        blk = sp[off[e]:off[e + 1]]
        assert (off[e + 1] - off[e]) % block_m == 0
        assert (blk >= 0).sum() == cnt_e[e]
        assert all(int(ids.reshape(-1)[p]) == e for p in blk[blk >= 0])
    # segments: joint histogram and padded lengths
    joint = {}
    for p in range(T * k):
        key = (int(ids.reshape(-1)[p]), int(ad[p // k]))
        joint[key] = joint.get(key, 0) + 1
    assert {(int(s[0]), int(s[1])): int(s[3]) for s in seg} == joint
    assert len(seg) == len(joint)
    for e in range(E):
        segs = [s for s in seg if s[0] == e]
        pos = off[e]
        for s in segs:
            assert s[2] == pos
            rows = sp[s[2]:s[2] + s[3]]
            assert all(int(ad[p // k]) == s[1] for p in rows)
            pad = sp[s[2] + s[3]: s[2] + -(-s[3] // seg_pad) * seg_pad]
            assert np.all(pad == -1)
            pos += -(-s[3] // seg_pad) * seg_pad
        assert off[e + 1] == off[e] + -(-(pos - off[e]) // block_m) * block_m
    return out


@pytest.mark.parametrize("seg_pad,block_m", [(1, 1), (1, 16), (16, 16), (16, 128), (4, 32)])
@pytest.mark.parametrize("name", ["tiny", "decode", "fg", "stress_distinct", "stress_same"])
def test_align_properties(name, seg_pad, block_m):
    w = configs.WORKLOADS[name]
    L = configs.make_logits(w, 1).numpy()
    ids, _ = oracle.route(L, w.topk)
    ad = configs.make_adapter_ids(w, 1).numpy()
    _check_align(ids, ad, w.n_experts, w.n_adapters, seg_pad, block_m)


def test_align_prefill_and_no_adapter():
    w = configs.WORKLOADS["prefill"]
    ids, _ = oracle.route(configs.make_logits(w, 0).numpy(), w.topk)
    ad = configs.make_adapter_ids(w, 0).numpy().copy()
    ad[::7] = -1
    _check_align(ids, ad, w.n_experts, w.n_adapters, 16, 128)


def test_align_empty_and_rejects():
    out = oracle.align(np.zeros((0, 2), np.int32), np.zeros(0, np.int32), 4, 2, 1, 16)
    assert out["sorted_pairs"].size == 0 and out["n_seg"] == 0
    assert out["expert_offsets"].tolist() == [0] * 5
    with pytest.raises(oracle.OracleError):
        oracle.align(np.array([[0, 5]], np.int32), np.array([0], np.int32), 4, 2, 1, 1)
    with pytest.raises(oracle.OracleError):
        oracle.align(np.array([[0, 1]], np.int32), np.array([2], np.int32), 4, 2, 1, 1)


# ----------------------------------------------------------------------------- forward

def test_forward_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    inp = {k: np.array(g[k], np.float64) for k in ("x", "W1", "W2", "A1", "B1", "A2", "B2")}
    inp["logits"] = np.array(g["logits"], np.float32)
    inp["adapter_ids"] = np.array(g["adapter_ids"], np.int32)
    y = oracle.forward(inp, g["dims"]["topk"])
    np.testing.assert_allclose(y, g["y"], rtol=g["tol"], atol=0)


def test_merged_weight_identity():
    """x(W + AB) written as stored matrices W' = W + B A must equal the LoRA form."""
    w = TINY
    inp = _f64_inputs(w, 0, b_scale=10.0)
    y = oracle.forward(inp, w.topk)
    ad = inp["adapter_ids"]
    ymerged = np.zeros_like(y)
    for a in range(w.n_adapters):
        m = dict(inp)
        m["W1"] = inp["W1"] + np.einsum("enq,eqc->enc", inp["B1"][a], inp["A1"][a])
        m["W2"] = inp["W2"] + np.einsum("emq,eqi->emi", inp["B2"][a], inp["A2"][a])
        m["adapter_ids"] = np.full(w.T, -1, np.int32)
        rows = np.nonzero(ad == a)[0]
        if rows.size:
            ymerged[rows] = oracle.forward(m, w.topk, tokens=rows)
    assert np.max(np.abs(y - ymerged)) <= 1e-12 * np.max(np.abs(y))
    # the LoRA terms are not negligible here, so the identity has teeth
    plain = dict(inp)
    plain["adapter_ids"] = np.full(w.T, -1, np.int32)
    assert np.max(np.abs(y - oracle.forward(plain, w.topk))) > 0.1 * np.max(np.abs(y))


def test_b_zero_is_plain_moe():
    w = TINY
    inp = _f64_inputs(w, 1)
    inp["B1"] = np.zeros_like(inp["B1"])
    inp["B2"] = np.zeros_like(inp["B2"])
    y = oracle.forward(inp, w.topk)
    plain = dict(inp)
    plain["adapter_ids"] = np.full(w.T, -1, np.int32)
    np.testing.assert_array_equal(y, oracle.forward(plain, w.topk))
    shuffled = dict(inp)
    shuffled["adapter_ids"] = inp["adapter_ids"][::-1].copy()
    np.testing.assert_array_equal(y, oracle.forward(shuffled, w.topk))


def test_one_adapter_batched_equals_per_token():
    w = TINY
    inp = _f64_inputs(w, 2)
    inp["adapter_ids"] = np.full(w.T, 3, np.int32)
    y = oracle.forward(inp, w.topk)
    for t in range(w.T):
        one = dict(inp)
        one["x"] = inp["x"][t:t + 1]
        one["logits"] = inp["logits"][t:t + 1]
        one["adapter_ids"] = inp["adapter_ids"][t:t + 1]
        np.testing.assert_allclose(oracle.forward(one, w.topk)[0], y[t], rtol=1e-12, atol=0)


def test_token_permutation():
    w = TINY
    inp = _f64_inputs(w, 3)
    y = oracle.forward(inp, w.topk)
    perm = np.random.default_rng(0).permutation(w.T)
    p = dict(inp)
    for kname in ("x", "logits", "adapter_ids"):
        p[kname] = inp[kname][perm].copy()
    np.testing.assert_array_equal(oracle.forward(p, w.topk), y[perm])
    # token subsets give the same rows
    np.testing.assert_array_equal(oracle.forward(inp, w.topk, tokens=perm[:5]), y[perm[:5]])


@pytest.mark.parametrize("dtype", [torch.float64, torch.bfloat16])
def test_single_expert_dense_ffn_vs_numpy(dtype):
    w = TINY.with_(n_experts=1, topk=1)
    d = configs.make_inputs(w, 4, dtype=dtype, b_scale=10.0)
    d["adapter_ids"][::5] = -1
    y = oracle.forward(d, 1)
    f = {k: v.double().numpy() if hasattr(v, "double") else v for k, v in d.items()}
    ad = d["adapter_ids"].numpy()
    ref = np.zeros_like(y)
    for a in np.unique(ad):
        rows = np.nonzero(ad == a)[0]
        aa = int(a)
        ref[rows] = _ffn_numpy(f["x"][rows], f["W1"][0], f["W2"][0],
                               f["A1"][max(aa, 0), 0], f["B1"][max(aa, 0), 0],
                               f["A2"][max(aa, 0), 0], f["B2"][max(aa, 0), 0], aa)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-14 * np.abs(ref).max())


def test_k_equals_E_combine_vs_numpy():
    w = TINY.with_(n_experts=4, topk=4)
    inp = _f64_inputs(w, 5, b_scale=10.0)
    y = oracle.forward(inp, w.topk)
    probs = scipy.special.softmax(inp["logits"].astype(np.float64), axis=1)
    ref = np.zeros_like(y)
    for t in range(w.T):
        a = int(inp["adapter_ids"][t])
        for e in range(w.n_experts):
            ref[t] += probs[t, e] * _ffn_numpy(inp["x"][t:t + 1], inp["W1"][e], inp["W2"][e],
                                               inp["A1"][a, e], inp["B1"][a, e], inp["A2"][a, e],
                                               inp["B2"][a, e], a)[0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-13 * np.abs(ref).max())


def test_zero_input_and_down_linearity():
    w = TINY
    inp = _f64_inputs(w, 6)
    z = dict(inp)
    z["x"] = np.zeros_like(inp["x"])
    assert np.all(oracle.forward(z, w.topk) == 0.0)
    y = oracle.forward(inp, w.topk)
    s = dict(inp)
    s["W2"] = 2.0 * inp["W2"]
    s["B2"] = 2.0 * inp["B2"]
    np.testing.assert_array_equal(oracle.forward(s, w.topk), 2.0 * y)


def test_forward_rejects_bad_adapter_and_logits():
    w = TINY
    inp = _f64_inputs(w, 0)
    bad = dict(inp)
    bad["adapter_ids"] = inp["adapter_ids"].copy()
    bad["adapter_ids"][3] = w.n_adapters
    with pytest.raises(oracle.OracleError):
        oracle.forward(bad, w.topk)
    bad = dict(inp)
    bad["logits"] = inp["logits"].copy()
    bad["logits"][0, 0] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.forward(bad, w.topk)


# ----------------------------------------------------------------------------- FP8 weights

# Values the OCP 8-bit floating point format fixes for E4M3 (bias 7, 3 mantissa bits, no
# infinities): zeros, the smallest subnormal 2^-9, the largest subnormal 7 * 2^-9, the smallest
# normal 2^-6, 1, 2, the largest finite 448, and the NaN encodings S.1111.111.
FP8_SPEC = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x40: 2.0, 0x39: 1.125, 0x3F: 1.875, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0,
            0xFE: -448.0}


def test_fp8_decode_spec_values():
    v = oracle.fp8e4m3_decode(np.arange(256))
    for code, want in FP8_SPEC.items():
        assert v[code] == want and np.signbit(v[code]) == np.signbit(want), hex(code)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and int(np.isnan(v).sum()) == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E increase"
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_fp8_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = oracle.fp8e4m3_decode(codes.numpy())
    same = (v == ref) | (np.isnan(v) & np.isnan(ref))
    assert same.all()


def test_fp8_forward_equals_dequantized_weights():
    """The E4M3 reader (codes times per-row scales) against the float64 path on the decoded
    weights, which the pins above already fix."""
    w = configs.Workload("fp8_tiny", 12, 256, 384, 6, 2, 3, 16)
    d = configs.make_inputs_fp8(w, 5)
    deq = dict(d)
    for name in ("W1", "W2"):
        deq[name] = oracle.fp8e4m3_decode(d[name].numpy()) * d[name + "_scale"].double().numpy()[..., None]
        del deq[name + "_scale"]
    y8 = oracle.forward(d, w.topk)
    y64 = oracle.forward(deq, w.topk)
    np.testing.assert_allclose(y8, y64, rtol=1e-12, atol=1e-15 * np.abs(y64).max())
    assert np.abs(y64).max() > 0


def test_fp8_quantized_rows_reproduce_weights():
    """The input preparation: decoded codes times the row scale stay within one E4M3 rounding
    (relative 2^-4) of the bf16 weights, and every row's largest magnitude maps to 448."""
    w = configs.Workload("fp8_q", 4, 128, 128, 3, 1, 2, 8)
    W = configs.make_inputs(w, 1)["W1"]
    codes, scale = configs.quantize_rows_e4m3(W)
    back = oracle.fp8e4m3_decode(codes.numpy()) * scale.double().numpy()[..., None]
    Wf = W.double().numpy()
    err = np.abs(back - Wf)
    assert np.all(err <= 2.0 ** -4 * np.abs(Wf) + 2.0 ** -9 * scale.double().numpy()[..., None])
    assert np.all(np.abs(oracle.fp8e4m3_decode(codes.numpy())).max(axis=-1) == 448.0)


# ----------------------------------------------------------------------------- dense multi-LoRA

def _sgmv_inputs(T, K, N, nA, r, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(T, K, generator=g) * 0.5).to(dtype)
    A = (torch.randn(nA, r, K, generator=g) * 0.1).to(dtype)
    B = (torch.randn(nA, N, r, generator=g) * 0.1).to(dtype)
    y = torch.randn(T, N, generator=g).to(dtype)
    ad = torch.randint(-1, nA, (T,), generator=g, dtype=torch.int32)
    return x, A, B, y, ad


@pytest.mark.parametrize("dtype", [torch.float64, torch.bfloat16])
def test_sgmv_vs_numpy_merged_weight(dtype):
    """Per token, y + x (B_a A_a)^T with the merged r-rank update formed by numpy matmul."""
    x, A, B, y, ad = _sgmv_inputs(37, 96, 80, 5, 8, 0, dtype)
    out = oracle.sgmv(x, A, B, y, ad)
    xn, An, Bn, yn = (t.double().numpy() for t in (x, A, B, y))
    for t in range(x.shape[0]):
        a = int(ad[t])
        want = yn[t] if a < 0 else yn[t] + xn[t] @ (Bn[a] @ An[a]).T
        np.testing.assert_allclose(out[t], want, rtol=1e-12, atol=1e-12)


def test_sgmv_no_adapter_and_zero_b():
    x, A, B, y, ad = _sgmv_inputs(20, 64, 48, 3, 16, 1)
    ad[:] = -1
    assert np.array_equal(oracle.sgmv(x, A, B, y, ad), y.numpy())
    ad2 = torch.zeros_like(ad)
    assert np.array_equal(oracle.sgmv(x, A, torch.zeros_like(B), y, ad2), y.numpy())


def test_sgmv_onto_zero_is_shrink_then_expand():
    """Onto y = 0 the output is the LoRA term alone, B_a (A_a x): the shrink-then-expand order
    (the test above multiplies the merged B_a A_a instead)."""
    T, h, I, nA, r = 9, 32, 16, 3, 8
    x, A, B, y, ad = _sgmv_inputs(T, h, 2 * I, nA, r, 2)
    z = oracle.sgmv(x, A, B, torch.zeros(T, 2 * I, dtype=torch.float64), ad)
    xn, An, Bn = x.numpy(), A.numpy(), B.numpy()
    for t in range(T):
        a = int(ad[t])
        want = np.zeros(2 * I) if a < 0 else Bn[a] @ (An[a] @ xn[t])
        np.testing.assert_allclose(z[t], want, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- router logits

@pytest.mark.parametrize("dtype", [torch.float64, torch.bfloat16])
def test_router_logits_vs_numpy(dtype):
    g = torch.Generator().manual_seed(11)
    x = torch.randn(23, 160, generator=g).to(dtype)
    W = torch.randn(12, 160, generator=g).to(dtype)
    got = oracle.router_logits(x, W)
    want = x.double().numpy() @ W.double().numpy().T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)

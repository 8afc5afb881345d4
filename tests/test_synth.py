"""The seeded input generator: published test vector, determinism, slicing, recipes. CPU only."""
import numpy as np
import torch

from synth import configs, gen


def test_splitmix64_published_vector():
    # SplitMix64 from state 0: first output 0xE220A8397B1DCDAF (Steele, Lea & Flood 2014;
    # the same stream as java.util.SplittableRandom's default mixing)
    assert gen.splitmix64_py(0, 1)[0] == 0xE220A8397B1DCDAF


def test_tensor_hash_matches_python():
    h = gen.hash_range(7, 3, 1000, 64)
    ref = gen.splitmix64_py(gen.stream_key(7, 3), 1064)[1000:]
    assert [int(v) & gen.MASK64 for v in h.tolist()] == ref


def test_slices_are_independent_of_chunking():
    full = gen.normal((3000,), 1, 4, 0.02, torch.float64)
    part = torch.empty(1000, dtype=torch.float64)
    h = gen.hash_range(1, 4, 1000, 1000)
    part = gen._box_muller(h) * 0.02
    torch.testing.assert_close(full[1000:2000], part, rtol=0, atol=0)


def test_normal_moments_and_bf16_rounding():
    x = gen.normal((1 << 18,), 0, 3, 0.02, torch.float64)
    assert abs(float(x.mean())) < 3 * 0.02 / 512
    assert abs(float(x.std()) - 0.02) < 0.02 * 0.01
    xb = gen.normal((1 << 18,), 0, 3, 0.02, torch.bfloat16)
    torch.testing.assert_close(xb, x.float().bfloat16(), rtol=0, atol=0)


def test_adapter_recipes():
    w = configs.WORKLOADS["prefill"]
    ids = configs.make_adapter_ids(w, 0)
    assert ids.shape == (w.T,)
    runs = ids.view(-1, w.run)
    assert torch.all(runs == runs[:, :1])
    assert int(ids.min()) >= 0 and int(ids.max()) < w.n_adapters
    sd = configs.make_adapter_ids(configs.WORKLOADS["stress_distinct"], 0)
    assert len(set(sd.tolist())) == 1024
    ss = configs.make_adapter_ids(configs.WORKLOADS["stress_same"], 0)
    assert torch.all(ss == 0)
    dec = configs.make_adapter_ids(configs.WORKLOADS["decode"], 0)
    assert int(dec.min()) >= 0 and int(dec.max()) < 8


def test_zipf_frequencies():
    p = np.array([i ** -1.1 for i in range(1, 33)])
    p /= p.sum()
    ids = gen.zipf_run_ids(0, 9, 200000, 1, 32, 1.1).numpy()
    freq = np.bincount(ids, minlength=32) / ids.size
    assert np.max(np.abs(freq - p)) < 0.01


def test_hot_expert_logits():
    w = configs.WORKLOADS["fg"]
    L = configs.make_logits(w, 0)
    base = gen.normal((w.T, w.n_experts), 0, gen.TID_LOGITS, 1.0, torch.float32)
    diff = (L - base)[0]
    assert int((diff != 0).sum()) == 8
    assert torch.allclose(diff[diff != 0], torch.tensor(2.0), atol=1e-6)


def test_same_seed_same_bytes():
    w = configs.WORKLOADS["tiny"]
    a = configs.make_inputs(w, 0)
    b = configs.make_inputs(w, 0)
    c = configs.make_inputs(w, 1)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert not torch.equal(a["W1"], c["W1"])

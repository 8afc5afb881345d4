"""The layer's synthetic workloads: sizes, value distributions and routing structure.

Each workload is a fused MoE layer of E experts (gate_up h -> 2I, SiLU-and-mul, down I -> h)
with nA LoRA adapters of rank r on both projections, top-k routing. Values follow the
initialiser convention N(0, sigma=0.02) for activations and weights, N(0,1) router logits.
"""
from __future__ import annotations

import dataclasses

import torch

from . import gen


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hidden: int
    inter: int
    n_experts: int
    topk: int
    n_adapters: int
    rank: int
    adapters: str = "uniform"       # uniform | zipf_runs | distinct | same
    hot_experts: int = 0            # experts whose logits get +hot_bias
    hot_bias: float = 0.0
    sigma: float = 0.02             # x, W, A
    sigma_b: float = 0.02           # B
    run: int = 512                  # run length for zipf_runs
    zipf_s: float = 1.1

    @property
    def pairs(self) -> int:
        return self.T * self.topk

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 512, 8, 2, 4, 8, sigma_b=0.01),
    "decode": Workload("decode", 64, 4096, 11008, 16, 2, 8, 16),
    "prefill": Workload("prefill", 4096, 4096, 14336, 8, 2, 32, 64, adapters="zipf_runs"),
    "fg": Workload("fg", 256, 2048, 768, 128, 8, 64, 32, hot_experts=8, hot_bias=2.0),
    "stress_distinct": Workload("stress_distinct", 1024, 4096, 11008, 16, 2, 1024, 16, adapters="distinct"),
    "stress_same": Workload("stress_same", 1024, 4096, 11008, 16, 2, 1024, 16, adapters="same"),
}


def make_logits(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    L = gen.normal((w.T, w.n_experts), seed, gen.TID_LOGITS, 1.0, torch.float32, device)
    if w.hot_experts:
        hot = gen.seeded_permutation(seed, gen.TID_HOT, w.n_experts)[: w.hot_experts].long()
        L[:, hot.to(device)] += torch.tensor(w.hot_bias, dtype=torch.float32, device=device)
    return L


def make_adapter_ids(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    if w.adapters == "uniform":
        return gen.uniform_ids(seed, gen.TID_ADAPTER, w.T, w.n_adapters, device)
    if w.adapters == "zipf_runs":
        return gen.zipf_run_ids(seed, gen.TID_ADAPTER, w.T, w.run, w.n_adapters, w.zipf_s, device)
    if w.adapters == "distinct":
        if w.n_adapters < w.T:
            raise ValueError("distinct adapters need n_adapters >= T")
        return gen.seeded_permutation(seed, gen.TID_ADAPTER, w.n_adapters, device)[: w.T].contiguous()
    if w.adapters == "same":
        return torch.zeros(w.T, dtype=torch.int32, device=device)
    raise ValueError(w.adapters)


WEIGHT_SHAPES = {
    "W1": lambda w: (w.n_experts, 2 * w.inter, w.hidden),
    "W2": lambda w: (w.n_experts, w.hidden, w.inter),
    "A1": lambda w: (w.n_adapters, w.n_experts, w.rank, w.hidden),
    "B1": lambda w: (w.n_adapters, w.n_experts, 2 * w.inter, w.rank),
    "A2": lambda w: (w.n_adapters, w.n_experts, w.rank, w.inter),
    "B2": lambda w: (w.n_adapters, w.n_experts, w.hidden, w.rank),
}
WEIGHT_TIDS = {"W1": gen.TID_W1, "W2": gen.TID_W2, "A1": gen.TID_A1, "B1": gen.TID_B1,
               "A2": gen.TID_A2, "B2": gen.TID_B2}


def make_inputs(w: Workload, seed: int, device="cpu", dtype=torch.bfloat16, b_scale: float = 1.0) -> dict:
    """All inputs of one layer call. Stored layouts (out x in, K contiguous):
    x[T][h], logits[T][E] f32, W1[E][2I][h], W2[E][h][I], A1[nA][E][r][h], B1[nA][E][2I][r],
    A2[nA][E][r][I], B2[nA][E][h][r], adapter_ids[T] int32."""
    d = {
        "x": gen.normal((w.T, w.hidden), seed, gen.TID_X, w.sigma, dtype, device),
        "logits": make_logits(w, seed, device),
        "adapter_ids": make_adapter_ids(w, seed, device),
    }
    for name, shp in WEIGHT_SHAPES.items():
        sig = w.sigma_b * b_scale if name in ("B1", "B2") else w.sigma
        d[name] = gen.normal(shp(w), seed, WEIGHT_TIDS[name], sig, dtype, device)
    return d


def quantize_rows_e4m3(W: torch.Tensor):
    """FP8 expert weights for the layer's FP8 entry point: every output row (last dim = input)
    gets the scale max|row| / 448 (448 is the largest E4M3 magnitude; an all-zero row gets 1),
    and its values divided by the scale are rounded to E4M3 by torch (round to nearest even).
    Returns (codes uint8, same shape; scales float32, shape without the last dim). Input
    preparation only: both the kernels and the oracle receive the codes and scales as given."""
    Wf = W.float()
    amax = Wf.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
    codes = (Wf / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def make_inputs_fp8(w: Workload, seed: int, device="cpu", b_scale: float = 1.0) -> dict:
    """make_inputs with W1 and W2 replaced by E4M3 codes and per-row scales (W1_scale [E][2I],
    W2_scale [E][h]); the other tensors are bf16 as in make_inputs."""
    d = make_inputs(w, seed, device=device, b_scale=b_scale)
    for name in ("W1", "W2"):
        codes, scale = quantize_rows_e4m3(d[name])
        d[name] = codes
        d[name + "_scale"] = scale
    return d


def input_bytes(w: Workload) -> int:
    n = w.T * w.hidden * 2 + w.T * w.n_experts * 4 + w.T * 4
    for shp in WEIGHT_SHAPES.values():
        s = 1
        for v in shp(w):
            s *= v
        n += 2 * s
    return n

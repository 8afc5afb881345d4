"""Seeded, counter-based synthetic inputs for the fused MoE + multi-LoRA layer.

This module only draws numbers. It holds none of the layer's arithmetic and is the one
piece of code that both the CPU oracle's tests and the HIP path's tests and benchmark use:
each side receives the same bytes, produced here.

Definition (every value is a pure function of (seed, tensor_id, element index)):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): state s advances by the golden gamma 0x9E3779B97F4A7C15 and each output is
  the "mix64" finaliser of the new state.
* Stream of a tensor: s0 = mix64((seed << 32) | tensor_id); element i takes the (i+1)-th
  output h_i = mix64(s0 + (i+1)*gamma) (arithmetic mod 2**64).
* Normal values: Box-Muller (Box & Muller 1958) on the two 32-bit halves of h_i,
  u1 = (hi + 1) / 2**32 in (0, 1], u2 = lo / 2**32 in [0, 1),
  n = sqrt(-2 ln u1) * cos(2 pi u2), evaluated in float64, times sigma.
* bf16 tensors: the float64 value rounded to float32, then to bfloat16, each step
  round-to-nearest-even (torch's conversions).

The torch implementation runs on CPU or GPU with the same integer steps; float64 Box-Muller
on two devices can differ in the last float64 bit, so a test that needs the same bytes on
both sides generates once and copies.
"""
from __future__ import annotations

import math

import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Fixed tensor ids of the layer's inputs.
TID_X, TID_LOGITS, TID_W1, TID_W2, TID_A1, TID_B1, TID_A2, TID_B2 = 1, 2, 3, 4, 5, 6, 7, 8
TID_ADAPTER, TID_HOT = 9, 10


def _s64(v: int) -> int:
    """Unsigned 64-bit constant as the signed int64 with the same bits."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_py(z: int) -> int:
    """SplitMix64 finaliser on a Python int (reference for the tensor version)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def splitmix64_py(state: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 from `state` (pure Python)."""
    out = []
    for _ in range(n):
        state = (state + GAMMA) & MASK64
        out.append(mix64_py(state))
    return out


def stream_key(seed: int, tensor_id: int) -> int:
    if not (0 <= seed < (1 << 32) and 0 <= tensor_id < (1 << 32)):
        raise ValueError("seed and tensor_id must fit in 32 bits")
    return mix64_py((seed << 32) | tensor_id)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(MIX2)
    return z ^ _lsr(z, 31)


def hash_range(seed: int, tensor_id: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """h_i for i in [start, start+count) as int64 bit patterns."""
    s0 = stream_key(seed, tensor_id)
    idx = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z = idx * _s64(GAMMA) + _s64(s0)
    return _mix64_t(z)


def _box_muller(h: torch.Tensor) -> torch.Tensor:
    hi = _lsr(h, 32).to(torch.float64)
    lo = (h & 0xFFFFFFFF).to(torch.float64)
    u1 = (hi + 1.0) * (1.0 / 4294967296.0)
    u2 = lo * (1.0 / 4294967296.0)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def uniform_u32(seed: int, tensor_id: int, count: int, device="cpu") -> torch.Tensor:
    """High 32 bits of h_i as int64 in [0, 2**32)."""
    return _lsr(hash_range(seed, tensor_id, 0, count, device), 32)


_CHUNK = 1 << 24      # elements per generation step on the CPU
_CHUNK_GPU = 1 << 27  # on a GPU: fewer, larger steps (the values do not depend on the chunking)


def normal_(out: torch.Tensor, seed: int, tensor_id: int, sigma: float, mean: float = 0.0) -> torch.Tensor:
    """Fill a contiguous tensor (bf16, f32 or f64, any device) with sigma * N(0,1) + mean."""
    if not out.is_contiguous():
        raise ValueError("normal_ needs a contiguous tensor")
    flat = out.view(-1)
    n = flat.numel()
    chunk = _CHUNK_GPU if out.device.type == "cuda" else _CHUNK
    for start in range(0, n, chunk):
        cnt = min(chunk, n - start)
        v = _box_muller(hash_range(seed, tensor_id, start, cnt, out.device)) * sigma + mean
        if out.dtype == torch.bfloat16:
            flat[start:start + cnt] = v.to(torch.float32).to(torch.bfloat16)
        else:
            flat[start:start + cnt] = v.to(out.dtype)
    return out


def normal(shape, seed: int, tensor_id: int, sigma: float, dtype=torch.bfloat16, device="cpu"):
    out = torch.empty(shape, dtype=dtype, device=device)
    return normal_(out, seed, tensor_id, sigma)


def seeded_permutation(seed: int, tensor_id: int, n: int, device="cpu") -> torch.Tensor:
    """Permutation of 0..n-1: indices ordered by (h_i as unsigned, i)."""
    h = hash_range(seed, tensor_id, 0, n, device)
    # order by unsigned value: flip the sign bit so signed order equals unsigned order
    key = h ^ _s64(1 << 63)
    return torch.sort(key, stable=True).indices.to(torch.int32)


def uniform_ids(seed: int, tensor_id: int, n: int, bound: int, device="cpu") -> torch.Tensor:
    """n ids in [0, bound): floor(hi32 * bound / 2**32) (multiply-shift)."""
    hi = uniform_u32(seed, tensor_id, n, device)
    return ((hi * bound) >> 32).to(torch.int32)


def zipf_run_ids(seed: int, tensor_id: int, n_tokens: int, run: int, n_adapters: int, s: float,
                 device="cpu") -> torch.Tensor:
    """Adapter id per token in runs of `run` tokens; each run's id is rank-1 of a draw from
    Zipf(s) over ranks 1..n_adapters (P(i) proportional to i**-s), by inverse CDF."""
    n_runs = (n_tokens + run - 1) // run
    w = torch.tensor([i ** -s for i in range(1, n_adapters + 1)], dtype=torch.float64)
    cdf = torch.cumsum(w, 0) / w.sum()
    hi = uniform_u32(seed, tensor_id, n_runs).to(torch.float64)
    u = (hi + 0.5) / 4294967296.0
    ranks = torch.searchsorted(cdf, u).clamp_(max=n_adapters - 1).to(torch.int32)
    ids = ranks.repeat_interleave(run)[:n_tokens]
    return ids.to(device)
